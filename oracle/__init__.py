"""ctypes wrapper around the plain-C CPU oracle (bitnet_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
bench's CPU-baseline leg.  The GPU library never imports, links or calls it.
All arrays are numpy arrays on the host.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bitnet_oracle.c")
_LIB = os.path.join(_HERE, "libbitnet_oracle.so")

def build_cmd(out: str) -> list[str]:
    return ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
            "-ffp-contract=off", "-fno-fast-math", _SRC, "-o", out, "-lm"]


def build() -> str:
    """Compile the oracle (always; cheap)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(build_cmd(tmp))
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.oracle_weight_scale.argtypes = [P, I64, I64, P]
        L.oracle_weight_scale.restype = ctypes.c_float
        L.oracle_pack.argtypes = [P, I64, I64, ctypes.c_float, ctypes.c_float, P]
        L.oracle_unpack.argtypes = [P, I64, I64, P]
        L.oracle_quant_act.argtypes = [P, I64, I64, P, P]
        L.oracle_linear.argtypes = [P, P, P, ctypes.c_float, I64, I64, I64, P, P]
        L.oracle_linear_bias.argtypes = [P, P, P, ctypes.c_float, P, I64, I64, I64, P, P]
        L.oracle_to_bf16.argtypes = [P, I64, P]
        L.oracle_rmsnorm_quant.argtypes = [P, P, ctypes.c_float, I64, I64, P, P]
        L.oracle_pack_grouped.argtypes = [P, I64, I64, I64, ctypes.c_float, P, P]
        L.oracle_swiglu_quant.argtypes = [P, P, I64, I64, P, P, P]
        L.oracle_quant_act_f32.argtypes = [P, I64, I64, P, P]
        L.oracle_pack_binary.argtypes = [P, I64, I64, P]
        L.oracle_linear_binary.argtypes = [P, P, P, ctypes.c_float, I64, I64, I64, P, P]
        L.oracle_pack_bitplanes.argtypes = [P, I64, I64, P]
        L.oracle_linear_bitplanes.argtypes = [P, P, P, ctypes.c_float, I64, I64, I64, P, P]
        L.oracle_linear_grouped.argtypes = [P, P, P, P, I64, P, I64, I64, I64, P, P]
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        L.oracle_get_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(lib().oracle_get_threads())


def weight_scale(w: np.ndarray) -> tuple[np.float32, np.ndarray]:
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    rows = np.empty(N, dtype=np.float64)
    s = lib().oracle_weight_scale(_p(w), N, K, _p(rows))
    return np.float32(s), rows


def pack(w: np.ndarray, eps: float = 1e-5) -> tuple[np.ndarray, np.float32]:
    """-> (packed uint8 [N][K/4], s_w)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    assert K % 4 == 0
    s_w, _ = weight_scale(w)
    out = np.empty((N, K // 4), dtype=np.uint8)
    lib().oracle_pack(_p(w), N, K, ctypes.c_float(eps), ctypes.c_float(s_w), _p(out))
    return out, s_w


def pack_grouped(w: np.ndarray, group: int, eps: float = 1e-5) -> tuple[np.ndarray, np.ndarray]:
    """Group-wise absmean scales (group = K: one per output channel) ->
    (packed uint8 [N][K/4], s_w fp32 [N][K/group])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    assert group > 0 and K % group == 0 and group % 4 == 0
    packed = np.empty((N, K // 4), dtype=np.uint8)
    s_w = np.empty((N, K // group), dtype=np.float32)
    lib().oracle_pack_grouped(_p(w), N, K, group, ctypes.c_float(eps), _p(s_w), _p(packed))
    return packed, s_w


def linear_grouped(q: np.ndarray, s_x: np.ndarray, packed: np.ndarray, s_w: np.ndarray, group: int,
                   bias: np.ndarray | None = None):
    """-> (acc int32 [M][N] (whole-row sums), y fp32 [M][N]) with group-wise scales."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    s_x = np.ascontiguousarray(s_x, dtype=np.float32)
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    s_w = np.ascontiguousarray(s_w, dtype=np.float32)
    M, K = q.shape
    N = packed.shape[0]
    assert packed.shape[1] * 4 == K and s_w.shape == (N, K // group)
    acc = np.empty((M, N), dtype=np.int32)
    y = np.empty((M, N), dtype=np.float32)
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
    lib().oracle_linear_grouped(_p(q), _p(s_x), _p(packed), _p(s_w), group,
                                None if bias is None else _p(bias), M, N, K, _p(acc), _p(y))
    return acc, y


def unpack(packed: np.ndarray, K: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    N = packed.shape[0]
    t = np.empty((N, K), dtype=np.int8)
    lib().oracle_unpack(_p(packed), N, K, _p(t))
    return t


def quant_act(x_bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """x_bits: uint16 [M][K] bf16 bit patterns -> (q int8 [M][K], s_x fp32 [M])."""
    x_bits = np.ascontiguousarray(x_bits).view(np.uint16)
    M, K = x_bits.shape
    q = np.empty((M, K), dtype=np.int8)
    s = np.empty(M, dtype=np.float32)
    lib().oracle_quant_act(_p(x_bits), M, K, _p(q), _p(s))
    return q, s


def rmsnorm_quant(x_bits: np.ndarray, gain: np.ndarray, eps: float) -> tuple[np.ndarray, np.ndarray]:
    """RMSNorm (gain g, eps) then absmax int8 of the normalized row:
    x_bits uint16 [M][K] bf16 patterns, gain fp32 [K] -> (q int8 [M][K], s_x fp32 [M])."""
    x_bits = np.ascontiguousarray(x_bits).view(np.uint16)
    gain = np.ascontiguousarray(gain, dtype=np.float32)
    M, K = x_bits.shape
    assert gain.shape == (K,)
    q = np.empty((M, K), dtype=np.int8)
    s = np.empty(M, dtype=np.float32)
    lib().oracle_rmsnorm_quant(_p(x_bits), _p(gain), ctypes.c_float(eps), M, K, _p(q), _p(s))
    return q, s


def pack_binary(w: np.ndarray) -> tuple[np.ndarray, np.float32]:
    """b1.0 binary weights: fp32 [N][K] -> (bits uint8 [N][K/8], s_w) with the
    absmean scale of the ternary path."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    assert K % 8 == 0
    bits = np.empty((N, K // 8), dtype=np.uint8)
    lib().oracle_pack_binary(_p(w), N, K, _p(bits))
    return bits, weight_scale(w)[0]


def linear_binary(q, s_x, bits, s_w, K: int | None = None):
    q = np.ascontiguousarray(q, dtype=np.int8)
    s_x = np.ascontiguousarray(s_x, dtype=np.float32)
    bits = np.ascontiguousarray(bits, dtype=np.uint8)
    M, K = q.shape
    N = bits.shape[0]
    acc = np.empty((M, N), dtype=np.int32)
    y = np.empty((M, N), dtype=np.float32)
    lib().oracle_linear_binary(_p(q), _p(s_x), _p(bits), ctypes.c_float(float(np.float32(s_w))), M, N, K,
                               _p(acc), _p(y))
    return acc, y


def pack_bitplanes(packed: np.ndarray, K: int) -> np.ndarray:
    """2-bit codes [N][K/4] -> sign / mask bitplanes uint8 [N][K/32][8]."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    N = packed.shape[0]
    assert K % 32 == 0 and packed.shape[1] == K // 4
    planes = np.empty((N, K // 32, 8), dtype=np.uint8)
    lib().oracle_pack_bitplanes(_p(packed), N, K, _p(planes))
    return planes


def linear_bitplanes(q, s_x, planes, s_w):
    q = np.ascontiguousarray(q, dtype=np.int8)
    s_x = np.ascontiguousarray(s_x, dtype=np.float32)
    planes = np.ascontiguousarray(planes, dtype=np.uint8)
    M, K = q.shape
    N = planes.shape[0]
    acc = np.empty((M, N), dtype=np.int32)
    y = np.empty((M, N), dtype=np.float32)
    lib().oracle_linear_bitplanes(_p(q), _p(s_x), _p(planes), ctypes.c_float(float(np.float32(s_w))), M, N, K,
                                  _p(acc), _p(y))
    return acc, y


def quant_act_f32(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """absmax int8 of fp32 rows: x [M][K] -> (q int8 [M][K], s_x fp32 [M])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.int8)
    s = np.empty(M, dtype=np.float32)
    lib().oracle_quant_act_f32(_p(x), M, K, _p(q), _p(s))
    return q, s


def swiglu_quant(g: np.ndarray, u: np.ndarray) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """a = fp32(silu(g) u), then absmax int8 of a: g, u fp32 [M][K] ->
    (a fp32 [M][K], q int8 [M][K], s_x fp32 [M])."""
    g = np.ascontiguousarray(g, dtype=np.float32)
    u = np.ascontiguousarray(u, dtype=np.float32)
    M, K = g.shape
    assert u.shape == (M, K)
    a = np.empty((M, K), dtype=np.float32)
    q = np.empty((M, K), dtype=np.int8)
    s = np.empty(M, dtype=np.float32)
    lib().oracle_swiglu_quant(_p(g), _p(u), M, K, _p(a), _p(q), _p(s))
    return a, q, s


def linear(q: np.ndarray, s_x: np.ndarray, packed: np.ndarray, s_w, K: int | None = None,
           bias: np.ndarray | None = None):
    """-> (acc int32 [M][N], y fp32 [M][N]); bias: fp32 [N] added after the rescale."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    s_x = np.ascontiguousarray(s_x, dtype=np.float32)
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    M, Kq = q.shape
    K = Kq if K is None else K
    N = packed.shape[0]
    assert packed.shape[1] * 4 == K and s_x.shape == (M,)
    acc = np.empty((M, N), dtype=np.int32)
    y = np.empty((M, N), dtype=np.float32)
    if bias is None:
        lib().oracle_linear(_p(q), _p(s_x), _p(packed), ctypes.c_float(float(s_w)),
                            M, N, K, _p(acc), _p(y))
    else:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        assert bias.shape == (N,)
        lib().oracle_linear_bias(_p(q), _p(s_x), _p(packed), ctypes.c_float(float(s_w)), _p(bias),
                                 M, N, K, _p(acc), _p(y))
    return acc, y


def to_bf16(y: np.ndarray) -> np.ndarray:
    """fp32 values -> bf16 bit patterns (uint16), nearest, ties to even."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint16)
    lib().oracle_to_bf16(_p(y), y.size, _p(out))
    return out
