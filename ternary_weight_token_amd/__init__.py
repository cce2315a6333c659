"""Python binding of libbitnet.so, the gfx950 BitNet b1.58 BitLinear forward.

Argument marshalling only: torch tensors (device memory) are turned into raw
pointers and sizes, the current torch stream into a hipStream_t, and a nonzero
status into an exception.  Every step of the computation runs in the library's
HIP kernels; there is no fallback.  The function names are those of the C ABI
(include/bitnet.h).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbitnet.so")

_lib = None


class BitnetError(RuntimeError):
    pass


class _LinearDesc(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("s_x", ctypes.c_void_p), ("packed", ctypes.c_void_p),
                ("s_w", ctypes.c_void_p), ("y", ctypes.c_void_p), ("acc", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("w_group", ctypes.c_int64),
                ("bias", ctypes.c_void_p), ("y_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class _FusedDesc(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("packed", ctypes.c_void_p), ("s_w", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("acc", ctypes.c_void_p), ("q", ctypes.c_void_p),
                ("s_x", ctypes.c_void_p), ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("norm_gain", ctypes.c_void_p), ("norm_eps", ctypes.c_float),
                ("x_f32", ctypes.c_void_p), ("packed_up", ctypes.c_void_p), ("s_w_up", ctypes.c_void_p),
                ("weight_fmt", ctypes.c_int32), ("y_dtype", ctypes.c_int32), ("bias", ctypes.c_void_p)]


class _QuantDesc(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("q", ctypes.c_void_p), ("s_x", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("K", ctypes.c_int64)]


def lib() -> ctypes.CDLL:
    """Load libbitnet.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python ternary_weight_token_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.bitnet_status_str.argtypes = [I]
        L.bitnet_status_str.restype = ctypes.c_char_p
        L.bitnet_last_error.restype = ctypes.c_char_p
        L.bitnet_version.restype = I
        L.bitnet_pack_workspace_bytes.argtypes = [I64, I64]
        L.bitnet_pack_workspace_bytes.restype = ctypes.c_size_t
        L.bitnet_pack_weights.argtypes = [P, I64, I64, ctypes.c_float, P, P, P, ctypes.c_size_t, P]
        L.bitnet_pack_weights_noalloc.argtypes = [P, I64, I64, ctypes.c_float, P, P, P]
        L.bitnet_quant_act.argtypes = [P, I64, I64, P, P, P]
        L.bitnet_rmsnorm_quant_act.argtypes = [P, P, ctypes.c_float, I64, I64, P, P, P]
        L.bitnet_swiglu_quant_act.argtypes = [P, P, I64, I64, P, P, P]
        L.bitnet_linear.argtypes = [P, P, P, P, I64, I64, I64, P, P, P]
        L.bitnet_linear_select.argtypes = [P, P, P, P, I64, I64, I64, P, P, I, P]
        L.bitnet_linear_ex.argtypes = [P, P, P, P, I64, I64, I64, I64, P, P, I, P, I, P]
        L.bitnet_pack_weights_grouped.argtypes = [P, I64, I64, I64, ctypes.c_float, P, P, P]
        L.bitnet_pack_weights_binary.argtypes = [P, I64, I64, P, P, P, ctypes.c_size_t, P]
        L.bitnet_pack_bitplanes.argtypes = [P, I64, I64, P, P]
        L.bitnet_linear_bits.argtypes = [P, P, P, I, P, I64, I64, I64, P, P, I, P]
        L.bitnet_grouped_plan_bytes.argtypes = [I, I, P]
        L.bitnet_grouped_plan_bytes.restype = ctypes.c_size_t
        L.bitnet_grouped_plan_linear.argtypes = [P, I, P, ctypes.c_size_t]
        L.bitnet_grouped_plan_quant.argtypes = [P, I, P, ctypes.c_size_t]
        L.bitnet_linear_grouped.argtypes = [P, P, P]
        L.bitnet_quant_act_grouped.argtypes = [P, P, P]
        L.bitnet_grouped_plan_fused_bytes.argtypes = [I, P]
        L.bitnet_grouped_plan_fused_bytes.restype = ctypes.c_size_t
        L.bitnet_grouped_plan_fused.argtypes = [P, I, P, ctypes.c_size_t]
        L.bitnet_linear_fused_grouped.argtypes = [P, P, P]
        L.bitnet_probe_stream_read.argtypes = [P, ctypes.c_size_t, I64, ctypes.c_uint32, P, P]
        L.bitnet_probe_mfma_i8.argtypes = [I64, I64, ctypes.c_uint32, P, P]
        L.bitnet_probe_mfma_i8_ops.argtypes = [I64, I64]
        L.bitnet_probe_mfma_i8_ops.restype = ctypes.c_double
        for f in ("bitnet_probe_stream_read", "bitnet_probe_mfma_i8",
                  "bitnet_pack_weights", "bitnet_pack_weights_noalloc", "bitnet_pack_weights_grouped", "bitnet_quant_act", "bitnet_rmsnorm_quant_act", "bitnet_swiglu_quant_act", "bitnet_pack_weights_binary", "bitnet_pack_bitplanes", "bitnet_linear_bits", "bitnet_linear", "bitnet_linear_select", "bitnet_linear_ex",
                  "bitnet_grouped_plan_linear", "bitnet_grouped_plan_quant", "bitnet_grouped_plan_fused",
                  "bitnet_linear_grouped", "bitnet_quant_act_grouped", "bitnet_linear_fused_grouped"):
            getattr(L, f).restype = I
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        L = lib()
        raise BitnetError(f"{L.bitnet_status_str(status).decode()} "
                          f"({L.bitnet_last_error().decode()})")


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(t: torch.Tensor, dtype, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _arg(t: torch.Tensor, dtype, shape, name: str) -> None:
    """A device tensor of this dtype and shape (the kernels trust the sizes they are given)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    _dev(t, dtype, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _same_device(name: str, *ts) -> None:
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"{name}: every tensor of a problem must be on one device")


def bitnet_pack_workspace_bytes(N: int, K: int) -> int:
    return int(lib().bitnet_pack_workspace_bytes(N, K))


def bitnet_pack_weights(w: torch.Tensor, eps: float, packed: torch.Tensor, s_w: torch.Tensor,
                        workspace: torch.Tensor, stream=None) -> None:
    """w fp32 [N][K] -> packed uint8 [N][K/4], s_w fp32 [1]."""
    _dev(w, torch.float32, "w"); _dev(packed, torch.uint8, "packed"); _dev(s_w, torch.float32, "s_w")
    N, K = w.shape
    if packed.shape != (N, K // 4) or s_w.numel() != 1:
        raise ValueError("packed must be [N][K/4] and s_w [1]")
    _check(lib().bitnet_pack_weights(_ptr(w), N, K, ctypes.c_float(eps), _ptr(packed), _ptr(s_w),
                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream)))


PACK_NOALLOC_MAX_ROWS = 262144


def bitnet_pack_weights_noalloc(w: torch.Tensor, eps: float, packed: torch.Tensor, s_w: torch.Tensor,
                                stream=None) -> None:
    """bitnet_pack_weights with the library's own per-GPU scratch (no workspace, no
    allocation); N <= PACK_NOALLOC_MAX_ROWS; calls overlapping on one GPU race."""
    _dev(w, torch.float32, "w"); _dev(packed, torch.uint8, "packed"); _dev(s_w, torch.float32, "s_w")
    N, K = w.shape
    if packed.shape != (N, K // 4) or s_w.numel() != 1:
        raise ValueError("packed must be [N][K/4] and s_w [1]")
    _check(lib().bitnet_pack_weights_noalloc(_ptr(w), N, K, ctypes.c_float(eps), _ptr(packed), _ptr(s_w),
                                             _stream(stream)))


def bitnet_quant_act(x: torch.Tensor, q: torch.Tensor, s_x: torch.Tensor, stream=None) -> None:
    """x bf16 [M][K] -> q int8 [M][K], s_x fp32 [M]."""
    _dev(x, torch.bfloat16, "x"); _dev(q, torch.int8, "q"); _dev(s_x, torch.float32, "s_x")
    M, K = x.shape
    if q.shape != (M, K) or s_x.shape != (M,):
        raise ValueError("q must be [M][K] and s_x [M]")
    _check(lib().bitnet_quant_act(_ptr(x), M, K, _ptr(q), _ptr(s_x), _stream(stream)))


def bitnet_rmsnorm_quant_act(x: torch.Tensor, gain: torch.Tensor, eps: float, q: torch.Tensor,
                             s_x: torch.Tensor, stream=None) -> None:
    """x bf16 [M][K], gain fp32 [K] -> q int8 [M][K], s_x fp32 [M] of the RMSNorm-ed rows."""
    _dev(x, torch.bfloat16, "x"); _dev(gain, torch.float32, "gain")
    _dev(q, torch.int8, "q"); _dev(s_x, torch.float32, "s_x")
    M, K = x.shape
    if gain.shape != (K,) or q.shape != (M, K) or s_x.shape != (M,):
        raise ValueError("gain must be [K], q [M][K] and s_x [M]")
    _check(lib().bitnet_rmsnorm_quant_act(_ptr(x), _ptr(gain), ctypes.c_float(eps), M, K, _ptr(q), _ptr(s_x),
                                          _stream(stream)))


def bitnet_swiglu_quant_act(gate: torch.Tensor, up: torch.Tensor, q: torch.Tensor, s_x: torch.Tensor,
                            stream=None) -> None:
    """gate, up fp32 [M][K] -> q int8 [M][K], s_x fp32 [M] of a = silu(gate) up."""
    _dev(gate, torch.float32, "gate"); _dev(up, torch.float32, "up")
    _dev(q, torch.int8, "q"); _dev(s_x, torch.float32, "s_x")
    M, K = gate.shape
    if up.shape != (M, K) or q.shape != (M, K) or s_x.shape != (M,):
        raise ValueError("up and q must be [M][K] like gate, s_x [M]")
    _check(lib().bitnet_swiglu_quant_act(_ptr(gate), _ptr(up), M, K, _ptr(q), _ptr(s_x), _stream(stream)))


def bitnet_linear(q: torch.Tensor, s_x: torch.Tensor, packed: torch.Tensor, s_w: torch.Tensor,
                  y: torch.Tensor, acc: torch.Tensor | None = None, stream=None) -> None:
    """q int8 [M][K], packed uint8 [N][K/4] -> y fp32 [M][N] (and acc int32 [M][N])."""
    _dev(q, torch.int8, "q"); _dev(s_x, torch.float32, "s_x"); _dev(packed, torch.uint8, "packed")
    _dev(s_w, torch.float32, "s_w"); _dev(y, torch.float32, "y")
    M, K = q.shape
    N = packed.shape[0]
    if packed.shape != (N, K // 4) or s_x.shape != (M,) or y.shape != (M, N):
        raise ValueError("shape mismatch")
    if acc is not None:
        _dev(acc, torch.int32, "acc")
        if acc.shape != (M, N):
            raise ValueError("acc must be [M][N]")
    _check(lib().bitnet_linear(_ptr(q), _ptr(s_x), _ptr(packed), _ptr(s_w), M, N, K, _ptr(y),
                               _ptr(acc), _stream(stream)))


KERNEL_AUTO, KERNEL_GEMV, KERNEL_GEMM, KERNEL_GENERIC = 0, 1, 2, 3


def bitnet_linear_select(q: torch.Tensor, s_x: torch.Tensor, packed: torch.Tensor, s_w: torch.Tensor,
                         y: torch.Tensor, acc: torch.Tensor | None, kernel: int, stream=None) -> None:
    """bitnet_linear with an explicit kernel choice (0 auto, 1 GEMV, 2 GEMM, 3 general)."""
    _dev(q, torch.int8, "q"); _dev(s_x, torch.float32, "s_x"); _dev(packed, torch.uint8, "packed")
    _dev(s_w, torch.float32, "s_w"); _dev(y, torch.float32, "y")
    M, K = q.shape
    N = packed.shape[0]
    if packed.shape != (N, K // 4) or s_x.shape != (M,) or y.shape != (M, N):
        raise ValueError("shape mismatch")
    if acc is not None:
        _dev(acc, torch.int32, "acc")
        if acc.shape != (M, N):
            raise ValueError("acc must be [M][N]")
    _check(lib().bitnet_linear_select(_ptr(q), _ptr(s_x), _ptr(packed), _ptr(s_w), M, N, K, _ptr(y),
                                      _ptr(acc), int(kernel), _stream(stream)))


BITNET_F32, BITNET_BF16 = 0, 1
_OUT_DTYPES = {torch.float32: BITNET_F32, torch.bfloat16: BITNET_BF16}


def bitnet_linear_ex(q: torch.Tensor, s_x: torch.Tensor, packed: torch.Tensor, s_w: torch.Tensor,
                     bias: torch.Tensor | None, y: torch.Tensor, acc: torch.Tensor | None = None,
                     kernel: int = 0, stream=None, w_group: int = 0) -> None:
    """bitnet_linear_select with an optional fp32 bias [N], y in fp32 or bf16 [M][N], and
    weight scales per tensor (w_group = 0, s_w [1]) or per group of w_group weights
    (s_w [N][K / w_group]; w_group = K: per output channel)."""
    _dev(q, torch.int8, "q"); _dev(s_x, torch.float32, "s_x"); _dev(packed, torch.uint8, "packed")
    _dev(s_w, torch.float32, "s_w")
    if w_group and s_w.numel() != packed.shape[0] * (q.shape[1] // w_group):
        raise ValueError("s_w must hold N * K / w_group scales")
    if y.dtype not in _OUT_DTYPES:
        raise ValueError(f"y must be float32 or bfloat16, got {y.dtype}")
    _dev(y, y.dtype, "y")
    M, K = q.shape
    N = packed.shape[0]
    if packed.shape != (N, K // 4) or s_x.shape != (M,) or y.shape != (M, N):
        raise ValueError("shape mismatch")
    if bias is not None:
        _dev(bias, torch.float32, "bias")
        if bias.shape != (N,):
            raise ValueError("bias must be [N]")
    if acc is not None:
        _dev(acc, torch.int32, "acc")
        if acc.shape != (M, N):
            raise ValueError("acc must be [M][N]")
    _check(lib().bitnet_linear_ex(_ptr(q), _ptr(s_x), _ptr(packed), _ptr(s_w), int(w_group), M, N, K, _ptr(bias),
                                  _ptr(y), _OUT_DTYPES[y.dtype], _ptr(acc), int(kernel), _stream(stream)))


class GroupedPlan:
    """A grouped launch plan: host image + device copy (see bitnet_grouped_plan_*)."""

    def __init__(self, host: bytes, dev: torch.Tensor, kind: str, refs: list):
        self.host = ctypes.create_string_buffer(host, len(host))
        self.dev = dev
        self.kind = kind
        self._refs = refs  # keep the described tensors alive

    @property
    def variant(self) -> int:
        """The plan header's kernel variant (the sixth 32-bit field after magic, kind,
        count, total_blocks, block_threads, rows_per_block and lds_bytes)."""
        return int.from_bytes(self.host.raw[28:32], "little")

    @property
    def flags(self) -> int:
        """The plan header's flags (its last 8 bytes); bit 0: a problem with group-wise
        weight scales asks for its int32 acc."""
        return int.from_bytes(self.host.raw[56:64], "little")

    def launch(self, stream=None) -> None:
        f = {"linear": lib().bitnet_linear_grouped, "quant": lib().bitnet_quant_act_grouped,
             "fused": lib().bitnet_linear_fused_grouped}[self.kind]
        _check(f(ctypes.cast(self.host, ctypes.c_void_p), _ptr(self.dev), _stream(stream)))


def _out_args(y, bias, M, N, where):
    """y: fp32 or bf16 [M][N]; bias: fp32 [N] or None -> (y_dtype, bias pointer)."""
    if not isinstance(y, torch.Tensor) or y.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"{where}: y must be an fp32 or bf16 tensor")
    _arg(y, y.dtype, (M, N), f"{where}: y")
    if bias is not None:
        _arg(bias, torch.float32, (N,), f"{where}: bias")
    return (1 if y.dtype == torch.bfloat16 else 0), (0 if bias is None else bias.data_ptr())


def bitnet_grouped_plan_linear(problems, device=None) -> GroupedPlan:
    """problems: list of (q, s_x, packed, s_w, y, acc_or_None[, w_group[, bias]]); w_group
    as in bitnet_linear_ex (s_w [N][K / w_group] when it is nonzero); y fp32 or bf16;
    bias an fp32 [N] added after the rescale, or None."""
    arr = (_LinearDesc * len(problems))()
    refs = []
    for i, prob in enumerate(problems):
        q, s_x, packed, s_w, y, acc = prob[:6]
        w_group = int(prob[6]) if len(prob) > 6 and prob[6] is not None else 0
        bias = prob[7] if len(prob) > 7 else None
        if not isinstance(q, torch.Tensor) or q.dim() != 2 or not isinstance(packed, torch.Tensor) or packed.dim() != 2:
            raise ValueError(f"problem {i}: q must be [M][K] and packed [N][K/4]")
        M, K = q.shape
        N = packed.shape[0]
        _arg(q, torch.int8, (M, K), f"problem {i}: q")
        _arg(s_x, torch.float32, (M,), f"problem {i}: s_x")
        _arg(packed, torch.uint8, (N, K // 4), f"problem {i}: packed")
        if w_group < 0 or (w_group and K % w_group):
            raise ValueError(f"problem {i}: w_group must be 0 or divide K")
        _dev(s_w, torch.float32, f"problem {i}: s_w")
        if s_w.numel() != (N * (K // w_group) if w_group else 1):
            raise ValueError(f"problem {i}: s_w must hold {'N * K / w_group' if w_group else 'one'} scale(s)")
        y_dtype, bias_p = _out_args(y, bias, M, N, f"problem {i}")
        if acc is not None:
            _arg(acc, torch.int32, (M, N), f"problem {i}: acc")
        _same_device(f"problem {i}", q, s_x, packed, s_w, y, acc, bias)
        arr[i] = _LinearDesc(q.data_ptr(), s_x.data_ptr(), packed.data_ptr(), s_w.data_ptr(),
                             y.data_ptr(), 0 if acc is None else acc.data_ptr(), M, packed.shape[0], K, w_group,
                             bias_p, y_dtype, 0)
        refs.append((q, s_x, packed, s_w, y, acc, bias))
    n = lib().bitnet_grouped_plan_bytes(len(problems), 1, ctypes.cast(arr, ctypes.c_void_p))
    buf = ctypes.create_string_buffer(n)
    _check(lib().bitnet_grouped_plan_linear(ctypes.cast(arr, ctypes.c_void_p), len(problems),
                                            ctypes.cast(buf, ctypes.c_void_p), n))
    host = buf.raw
    dev = torch.frombuffer(bytearray(host), dtype=torch.uint8).to(device or problems[0][0].device)
    return GroupedPlan(host, dev, "linear", refs)


def bitnet_grouped_plan_quant(problems, device=None) -> GroupedPlan:
    """problems: list of (x, q, s_x)."""
    arr = (_QuantDesc * len(problems))()
    refs = []
    for i, (x, q, s_x) in enumerate(problems):
        if not isinstance(x, torch.Tensor) or x.dim() != 2:
            raise ValueError(f"problem {i}: x must be [M][K]")
        M, K = x.shape
        _arg(x, torch.bfloat16, (M, K), f"problem {i}: x")
        _arg(q, torch.int8, (M, K), f"problem {i}: q")
        _arg(s_x, torch.float32, (M,), f"problem {i}: s_x")
        _same_device(f"problem {i}", x, q, s_x)
        arr[i] = _QuantDesc(x.data_ptr(), q.data_ptr(), s_x.data_ptr(), M, K)
        refs.append((x, q, s_x))
    n = lib().bitnet_grouped_plan_bytes(len(problems), 0, ctypes.cast(arr, ctypes.c_void_p))
    buf = ctypes.create_string_buffer(n)
    _check(lib().bitnet_grouped_plan_quant(ctypes.cast(arr, ctypes.c_void_p), len(problems),
                                           ctypes.cast(buf, ctypes.c_void_p), n))
    host = buf.raw
    dev = torch.frombuffer(bytearray(host), dtype=torch.uint8).to(device or problems[0][0].device)
    return GroupedPlan(host, dev, "quant", refs)


def bitnet_grouped_plan_fused(problems, device=None) -> GroupedPlan:
    """problems: list of (x, packed, s_w, y, acc_or_None, q_or_None, s_x_or_None
    [, norm_gain, norm_eps[, bias]]).  x is a bf16 [1][K] row (quantized inside the
    launch, after an RMSNorm with the fp32 gain [K] when one is given) or an fp32 [1][K]
    row (quantized the same way, no norm).  packed and s_w are one matrix, or the pairs
    (packed_gate, packed_up) and (s_w_gate, s_w_up) of a SwiGLU feed-forward part,
    whose y gets fp32(silu(y_gate) y_up).  Weights as sign / mask bitplanes are given
    as [N][K/32][8] tensors (pack_bitplanes), every problem of the plan alike.  y is
    fp32 or bf16; bias an fp32 [N] added after the rescale (not on pairs) or None;
    bitplane plans take fp32 y and no bias."""
    arr = (_FusedDesc * len(problems))()
    refs = []
    for i, prob in enumerate(problems):
        x, packed, s_w, y, acc, q, s_x = prob[:7]
        gain, eps = (prob[7], float(prob[8])) if len(prob) > 7 and prob[7] is not None else (None, 0.0)
        bias = prob[9] if len(prob) > 9 else None
        if not isinstance(x, torch.Tensor) or x.dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("x must be a bf16 or fp32 tensor")
        if x.dim() != 2:
            raise ValueError(f"problem {i}: x must be [M][K]")
        M, K = x.shape
        _arg(x, x.dtype, (M, K), f"problem {i}: x")
        xp, xf = (x.data_ptr(), 0) if x.dtype == torch.bfloat16 else (0, x.data_ptr())
        pu = su = 0
        packed_up = s_w_up = None
        if isinstance(packed, (tuple, list)):
            packed, packed_up = packed
            s_w, s_w_up = s_w
        if not isinstance(packed, torch.Tensor) or packed.dim() not in (2, 3):
            raise ValueError(f"problem {i}: packed must be [N][K/4] (or bitplanes [N][K/32][8])")
        N = packed.shape[0]
        fmt = FMT_BITPLANES if packed.dim() == 3 else 0
        _arg(packed, torch.uint8, (N, K // 32, 8) if fmt else (N, K // 4), f"problem {i}: packed")
        _arg(s_w, torch.float32, (1,), f"problem {i}: s_w")
        if packed_up is not None:
            _arg(packed_up, torch.uint8, tuple(packed.shape), f"problem {i}: packed_up")
            _arg(s_w_up, torch.float32, (1,), f"problem {i}: s_w_up")
            pu, su = packed_up.data_ptr(), s_w_up.data_ptr()
            refs.append((packed_up, s_w_up))
        y_dtype, bias_p = _out_args(y, bias, M, N, f"problem {i}")
        if acc is not None:
            _arg(acc, torch.int32, (M, N), f"problem {i}: acc")
        if q is not None:
            _arg(q, torch.int8, (M, K), f"problem {i}: q")
        if s_x is not None:
            _arg(s_x, torch.float32, (M,), f"problem {i}: s_x")
        if gain is not None:
            _arg(gain, torch.float32, (K,), f"problem {i}: norm_gain")
        _same_device(f"problem {i}", x, packed, s_w, y, acc, q, s_x, gain, packed_up, s_w_up, bias)
        arr[i] = _FusedDesc(xp, packed.data_ptr(), s_w.data_ptr(), y.data_ptr(),
                            0 if acc is None else acc.data_ptr(), 0 if q is None else q.data_ptr(),
                            0 if s_x is None else s_x.data_ptr(), M, packed.shape[0], K,
                            0 if gain is None else gain.data_ptr(), eps, xf, pu, su, fmt, y_dtype, bias_p)
        refs.append((x, packed, s_w, y, acc, q, s_x, gain, bias))
    n = lib().bitnet_grouped_plan_fused_bytes(len(problems), ctypes.cast(arr, ctypes.c_void_p))
    buf = ctypes.create_string_buffer(n)
    _check(lib().bitnet_grouped_plan_fused(ctypes.cast(arr, ctypes.c_void_p), len(problems),
                                           ctypes.cast(buf, ctypes.c_void_p), n))
    host = buf.raw
    dev = torch.frombuffer(bytearray(host), dtype=torch.uint8).to(device or problems[0][0].device)
    return GroupedPlan(host, dev, "fused", refs)


# ----------------------------------------------------------------- conveniences

def pack_weights(w: torch.Tensor, eps: float = 1e-5, stream=None):
    """Allocate outputs and run bitnet_pack_weights -> (packed, s_w)."""
    N, K = w.shape
    packed = torch.empty((N, K // 4), dtype=torch.uint8, device=w.device)
    s_w = torch.empty(1, dtype=torch.float32, device=w.device)
    ws = torch.empty(max(1, bitnet_pack_workspace_bytes(N, K) // 8), dtype=torch.float64, device=w.device)
    bitnet_pack_weights(w, eps, packed, s_w, ws, stream)
    return packed, s_w


def rmsnorm_quant(x: torch.Tensor, gain: torch.Tensor, eps: float, stream=None):
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    s_x = torch.empty(M, dtype=torch.float32, device=x.device)
    bitnet_rmsnorm_quant_act(x, gain, eps, q, s_x, stream)
    return q, s_x


def swiglu_quant(gate: torch.Tensor, up: torch.Tensor, stream=None):
    M, K = gate.shape
    q = torch.empty((M, K), dtype=torch.int8, device=gate.device)
    s_x = torch.empty(M, dtype=torch.float32, device=gate.device)
    bitnet_swiglu_quant_act(gate, up, q, s_x, stream)
    return q, s_x


FMT_BINARY, FMT_BITPLANES = 1, 2


def pack_weights_binary(w: torch.Tensor, stream=None):
    """b1.0 binary packing -> (bits uint8 [N][K/8], s_w fp32 [1])."""
    _dev(w, torch.float32, "w")
    N, K = w.shape
    bits = torch.empty((N, K // 8), dtype=torch.uint8, device=w.device)
    s_w = torch.empty(1, dtype=torch.float32, device=w.device)
    ws = torch.empty(max(1, bitnet_pack_workspace_bytes(N, K) // 8), dtype=torch.float64, device=w.device)
    _check(lib().bitnet_pack_weights_binary(_ptr(w), N, K, _ptr(bits), _ptr(s_w), _ptr(ws), ws.numel() * 8,
                                            _stream(stream)))
    return bits, s_w


def pack_bitplanes(packed: torch.Tensor, K: int, stream=None) -> torch.Tensor:
    """2-bit packed [N][K/4] -> sign / mask bitplanes uint8 [N][K/32][8]."""
    _dev(packed, torch.uint8, "packed")
    N = packed.shape[0]
    if packed.shape != (N, K // 4):
        raise ValueError("packed must be [N][K/4]")
    planes = torch.empty((N, K // 32, 8), dtype=torch.uint8, device=packed.device)
    _check(lib().bitnet_pack_bitplanes(_ptr(packed), N, K, _ptr(planes), _stream(stream)))
    return planes


def bitnet_linear_bits(q, s_x, wbits, fmt: int, s_w, y, acc=None, kernel: int = 0, stream=None) -> None:
    """q int8 [M][K] against binary bits [N][K/8] or bitplanes [N][K/32][8] -> y fp32
    [M][N] (and acc int32 [M][N])."""
    _dev(q, torch.int8, "q"); _dev(s_x, torch.float32, "s_x"); _dev(wbits, torch.uint8, "wbits")
    _dev(s_w, torch.float32, "s_w"); _dev(y, torch.float32, "y")
    M, K = q.shape
    N = wbits.shape[0]
    if wbits.numel() != N * K // (8 if fmt == FMT_BINARY else 4) or y.shape != (M, N):
        raise ValueError("weights do not match K, or y is not [M][N]")
    if acc is not None:
        _arg(acc, torch.int32, (M, N), "acc")
    if s_x.shape != (M,) or s_w.numel() != 1:
        raise ValueError("s_x must be [M] and s_w [1]")
    _check(lib().bitnet_linear_bits(_ptr(q), _ptr(s_x), _ptr(wbits), int(fmt), _ptr(s_w), M, N, K, _ptr(y),
                                    _ptr(acc), int(kernel), _stream(stream)))


def linear_bits(q, s_x, wbits, fmt: int, s_w, want_acc: bool = False, kernel: int = 0, stream=None):
    """y (and acc) of q against binary bits [N][K/8] or bitplanes [N][K/32][8]."""
    M, K = q.shape
    N = wbits.shape[0]
    y = torch.empty((M, N), dtype=torch.float32, device=q.device)
    acc = torch.empty((M, N), dtype=torch.int32, device=q.device) if want_acc else None
    bitnet_linear_bits(q, s_x, wbits, fmt, s_w, y, acc, kernel, stream)
    return (y, acc) if want_acc else y


def pack_weights_grouped(w: torch.Tensor, group: int, eps: float = 1e-5, stream=None):
    """Group-wise absmean packing -> (packed uint8 [N][K/4], s_w fp32 [N][K/group])."""
    _dev(w, torch.float32, "w")
    N, K = w.shape
    packed = torch.empty((N, K // 4), dtype=torch.uint8, device=w.device)
    s_w = torch.empty((N, K // group if group else 0), dtype=torch.float32, device=w.device)
    _check(lib().bitnet_pack_weights_grouped(_ptr(w), N, K, int(group), ctypes.c_float(eps), _ptr(packed),
                                             _ptr(s_w), _stream(stream)))
    return packed, s_w


def quant_act(x: torch.Tensor, stream=None):
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    s_x = torch.empty(M, dtype=torch.float32, device=x.device)
    bitnet_quant_act(x, q, s_x, stream)
    return q, s_x


def linear(q, s_x, packed, s_w, want_acc: bool = False, stream=None, bias=None,
           out_dtype=torch.float32, kernel: int = 0, w_group: int = 0):
    M, K = q.shape
    N = packed.shape[0]
    y = torch.empty((M, N), dtype=out_dtype, device=q.device)
    acc = torch.empty((M, N), dtype=torch.int32, device=q.device) if want_acc else None
    if bias is None and out_dtype == torch.float32 and kernel == 0 and w_group == 0:
        bitnet_linear(q, s_x, packed, s_w, y, acc, stream)
    else:
        bitnet_linear_ex(q, s_x, packed, s_w, bias, y, acc, kernel, stream, w_group)
    return (y, acc) if want_acc else y


# ------------------------------------------------------------------ measurement probes
PROBE_KEY = 0x9E3779B9


def probe_stream_read(buf: torch.Tensor, sink: torch.Tensor, blocks: int = 2048, stream=None) -> None:
    """Read every byte of buf once (bitnet_probe_stream_read): the HBM streaming
    ceiling next to which the decode kernels are measured."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    _arg(sink, torch.int32, (1,), "sink")
    nbytes = buf.numel() * buf.element_size()
    _check(lib().bitnet_probe_stream_read(_ptr(buf), nbytes, int(blocks), PROBE_KEY, _ptr(sink), _stream(stream)))


def probe_mfma_i8(sink: torch.Tensor, blocks: int, iters: int, stream=None) -> float:
    """int8 MFMAs from registers only (bitnet_probe_mfma_i8); returns the int8
    operations of the launch."""
    _arg(sink, torch.int32, (1,), "sink")
    _check(lib().bitnet_probe_mfma_i8(int(blocks), int(iters), PROBE_KEY, _ptr(sink), _stream(stream)))
    return float(lib().bitnet_probe_mfma_i8_ops(int(blocks), int(iters)))
