"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point include/bitnet.h declares, and rejects invalid arguments
before enqueuing anything (no kernel is launched by any call in this file)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import ternary_weight_token_amd as tw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("bitnet.h", "bitnet_probe.h")]

OK, NULL, SHAPE, ALIGN, HIP, ARG = range(6)


def declared_functions():
    src = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"BITNET_API\s+[\w\s\*]+?\b(bitnet_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tw.LIB_PATH):
        from ternary_weight_token_amd import build
        build.build()
    return tw.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) == 27, names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for s in range(6):
        assert L.bitnet_status_str(s).decode().startswith("BITNET_")
    assert L.bitnet_version() == 100


def test_probes_reject_bad_arguments(L):
    p = ctypes.c_void_p(4096)  # never dereferenced: every call below fails its checks
    z = None
    sr, mf = L.bitnet_probe_stream_read, L.bitnet_probe_mfma_i8
    assert sr(z, 1024, 8, 1, p, z) == NULL
    assert sr(p, 1024, 8, 1, z, z) == NULL
    assert sr(p, 1000, 8, 1, p, z) == SHAPE          # bytes % 16
    assert sr(p, 0, 8, 1, p, z) == SHAPE
    assert sr(p, 1024, 0, 1, p, z) == SHAPE          # blocks
    assert sr(p, 1024, 65537, 1, p, z) == SHAPE
    assert sr(ctypes.c_void_p(4100), 1024, 8, 1, p, z) == ALIGN
    assert mf(8, 10, 1, z, z) == NULL
    assert mf(0, 10, 1, p, z) == SHAPE
    assert mf(8, (1 << 24) + 1, 1, p, z) == SHAPE
    assert mf(8, 10, 1, ctypes.c_void_p(4098), z) == ALIGN
    assert L.bitnet_probe_mfma_i8_ops(2, 3) == 2 * 8 * 8 * 3 * 2 * 16 * 16 * 64


def test_linear_rejects_bad_arguments(L):
    p = ctypes.c_void_p(256)  # never dereferenced: every call below fails its checks
    z = None
    # NULL pointers
    assert L.bitnet_linear(z, p, p, p, 1, 1, 64, p, z, z) == NULL
    assert L.bitnet_linear(p, p, p, p, 1, 1, 64, z, z, z) == NULL
    # shapes
    assert L.bitnet_linear(p, p, p, p, 1, 1, 6, p, z, z) == SHAPE
    assert L.bitnet_linear(p, p, p, p, 1, 1, 0, p, z, z) == SHAPE
    assert L.bitnet_linear(p, p, p, p, -1, 1, 64, p, z, z) == SHAPE
    assert L.bitnet_linear(p, p, p, p, 1, -5, 64, p, z, z) == SHAPE
    assert L.bitnet_linear(p, p, p, p, 1 << 31, 1, 64, p, z, z) == SHAPE
    # alignment of the fp32 / int32 arrays
    assert L.bitnet_linear(p, ctypes.c_void_p(257), p, p, 1, 1, 64, p, z, z) == ALIGN
    assert L.bitnet_linear(p, p, p, p, 1, 1, 64, ctypes.c_void_p(258), z, z) == ALIGN
    assert L.bitnet_linear(p, p, p, p, 1, 1, 64, p, ctypes.c_void_p(2), z) == ALIGN
    # empty problems are successful no-ops, even with NULL pointers
    assert L.bitnet_linear(z, z, z, z, 0, 5, 64, z, z, z) == OK
    assert L.bitnet_linear(z, z, z, z, 3, 0, 64, z, z, z) == OK


def test_linear_ex_rejects_bad_arguments(L):
    p = ctypes.c_void_p(256)  # never dereferenced: every call below fails its checks
    z = None
    F32, BF16 = 0, 1
    assert L.bitnet_linear_ex(p, p, p, p, 0, 1, 1, 64, z, p, 2, z, 0, z) == ARG       # unknown dtype
    assert L.bitnet_linear_ex(p, p, p, p, 0, 1, 1, 64, z, p, F32, z, 7, z) == ARG     # unknown kernel
    assert L.bitnet_linear_ex(p, p, p, p, 0, 1, 1, 64, ctypes.c_void_p(258), p, F32, z, 0, z) == ALIGN
    assert L.bitnet_linear_ex(p, p, p, p, 0, 1, 1, 64, z, ctypes.c_void_p(258), F32, z, 0, z) == ALIGN
    assert L.bitnet_linear_ex(p, p, p, p, 0, 1, 1, 64, z, ctypes.c_void_p(257), BF16, z, 0, z) == ALIGN
    assert L.bitnet_linear_ex(p, p, p, p, 0, 1, 1, 64, p, z, BF16, z, 0, z) == NULL
    assert L.bitnet_linear_ex(p, p, p, p, 0, 1, 1, 6, p, p, BF16, z, 0, z) == SHAPE
    # fast kernels need K % 64 == 0 (the general kernel, id 3, does not)
    assert L.bitnet_linear_ex(p, p, p, p, 0, 1, 1, 68, z, p, BF16, z, 1, z) == ALIGN
    assert L.bitnet_linear_ex(z, z, z, z, 0, 0, 5, 64, z, z, BF16, z, 0, z) == OK
    # weight-scale groups: a multiple of 4 dividing K; below K only kernels 0, 1, 3;
    # the GEMV also needs a multiple of 64
    assert L.bitnet_linear_ex(p, p, p, p, 6, 1, 1, 64, z, p, F32, z, 0, z) == SHAPE
    assert L.bitnet_linear_ex(p, p, p, p, 48, 1, 1, 128, z, p, F32, z, 0, z) == SHAPE
    assert L.bitnet_linear_ex(p, p, p, p, -4, 1, 1, 64, z, p, F32, z, 0, z) == SHAPE
    # group-wise scales: not on the MFMA decode kernel or the older GEMM tiles; on the
    # pipelined GEMM only without acc, K % 128 == 0 and G = 64 or a multiple of 128
    for kern in (4, 16, 20):
        assert L.bitnet_linear_ex(p, p, p, p, 64, 1, 1, 128, z, p, F32, z, kern, z) == ARG
    for kern in (2, 21, 22):
        assert L.bitnet_linear_ex(p, p, p, p, 64, 1, 1, 128, z, p, F32, p, kern, z) == ARG     # with acc
        assert L.bitnet_linear_ex(p, p, p, p, 192, 1, 1, 384, z, p, F32, z, kern, z) == ARG    # G = 192
        assert L.bitnet_linear_ex(p, p, p, p, 64, 1, 1, 192, z, p, F32, z, kern, z) == ARG     # K % 128
    assert L.bitnet_linear_ex(p, p, p, p, 32, 1, 1, 128, z, p, F32, z, 1, z) == ALIGN


def test_pack_grouped_rejects_bad_arguments(L):
    p = ctypes.c_void_p(256)
    z = None
    f = ctypes.c_float(1e-5)
    assert L.bitnet_pack_weights_grouped(p, 2, 64, 0, f, p, p, z) == SHAPE
    assert L.bitnet_pack_weights_grouped(p, 2, 64, 6, f, p, p, z) == SHAPE
    assert L.bitnet_pack_weights_grouped(p, 2, 64, 48, f, p, p, z) == SHAPE
    assert L.bitnet_pack_weights_grouped(z, 2, 64, 32, f, p, p, z) == NULL
    assert L.bitnet_pack_weights_grouped(p, 2, 64, 32, f, p, ctypes.c_void_p(258), z) == ALIGN
    assert L.bitnet_pack_weights_grouped(z, 0, 64, 32, f, z, z, z) == OK


def test_quant_and_pack_reject_bad_arguments(L):
    p = ctypes.c_void_p(256)
    z = None
    assert L.bitnet_quant_act(z, 1, 64, p, p, z) == NULL
    assert L.bitnet_quant_act(p, 1, 66, p, p, z) == SHAPE
    assert L.bitnet_quant_act(ctypes.c_void_p(257), 1, 64, p, p, z) == ALIGN
    assert L.bitnet_quant_act(z, 0, 64, z, z, z) == OK
    assert L.bitnet_pack_workspace_bytes(10, 64) == 80
    assert L.bitnet_pack_weights(z, 2, 64, ctypes.c_float(1e-5), p, p, p, 16, z) == NULL
    assert L.bitnet_pack_weights(p, 2, 62, ctypes.c_float(1e-5), p, p, p, 16, z) == SHAPE
    assert L.bitnet_pack_weights(p, 2, 64, ctypes.c_float(1e-5), p, p, p, 8, z) == ARG
    assert L.bitnet_pack_weights(p, 2, 64, ctypes.c_float(1e-5), p, p, ctypes.c_void_p(260), 16, z) == ALIGN


def test_grouped_plan_checks(L):
    D = tw._LinearDesc
    a16 = 4096
    good = D(a16, a16, a16, a16, a16, 0, 1, 100, 2560)
    arr = (D * 2)(good, D(a16, a16, a16, a16, a16, 0, 17, 100, 2560))
    n = L.bitnet_grouped_plan_bytes(2, 1, ctypes.cast(arr, ctypes.c_void_p))
    buf = ctypes.create_string_buffer(n)
    # M = 17 is beyond the grouped decode path
    assert L.bitnet_grouped_plan_linear(ctypes.cast(arr, ctypes.c_void_p), 2,
                                        ctypes.cast(buf, ctypes.c_void_p), n) == SHAPE
    arr2 = (D * 1)(D(a16 + 4, a16, a16, a16, a16, 0, 1, 100, 2560))
    assert L.bitnet_grouped_plan_linear(ctypes.cast(arr2, ctypes.c_void_p), 1,
                                        ctypes.cast(buf, ctypes.c_void_p), n) == ALIGN
    arr3 = (D * 1)(good)
    n3 = L.bitnet_grouped_plan_bytes(1, 1, ctypes.cast(arr3, ctypes.c_void_p))
    assert L.bitnet_grouped_plan_linear(ctypes.cast(arr3, ctypes.c_void_p), 1,
                                        ctypes.cast(buf, ctypes.c_void_p), n3 - 1) == ARG
    assert L.bitnet_grouped_plan_linear(ctypes.cast(arr3, ctypes.c_void_p), 1,
                                        ctypes.cast(buf, ctypes.c_void_p), n3) == OK
    # a linear plan is not a quant plan; a random buffer is not a plan
    dev = ctypes.c_void_p(4096)
    assert L.bitnet_quant_act_grouped(ctypes.cast(buf, ctypes.c_void_p), dev, None) == ARG
    junk = ctypes.create_string_buffer(128)
    assert L.bitnet_linear_grouped(ctypes.cast(junk, ctypes.c_void_p), dev, None) == ARG
    assert L.bitnet_linear_grouped(ctypes.cast(buf, ctypes.c_void_p), ctypes.c_void_p(4100), None) == ALIGN
    # the header records the block count: ceil(N / rows_per_block) * M
    hdr = (ctypes.c_uint32 * 8).from_buffer_copy(buf.raw[:32])
    assert hdr[5] > 0 and hdr[3] == (100 + hdr[5] - 1) // hdr[5]
    # a K whose staged q exceeds the LDS budget is walked in segments: accepted,
    # and the recorded LDS size stays within 64 KiB
    arr4 = (D * 1)(D(a16, a16, a16, a16, a16, 0, 1, 100, 64 * 1000))
    n4 = L.bitnet_grouped_plan_bytes(1, 1, ctypes.cast(arr4, ctypes.c_void_p))
    buf4 = ctypes.create_string_buffer(n4)
    assert L.bitnet_grouped_plan_linear(ctypes.cast(arr4, ctypes.c_void_p), 1,
                                        ctypes.cast(buf4, ctypes.c_void_p), n4) == OK
    hdr4 = (ctypes.c_uint32 * 8).from_buffer_copy(buf4.raw[:32])
    assert 0 < hdr4[6] <= 64 * 1024
    # any M > 1 selects the MFMA variant: one block per 256 rows for all M tokens
    arr5 = (D * 2)(D(a16, a16, a16, a16, a16, 0, 1, 300, 2560), D(a16, a16, a16, a16, a16, 0, 5, 200, 2560))
    n5 = L.bitnet_grouped_plan_bytes(2, 1, ctypes.cast(arr5, ctypes.c_void_p))
    buf5 = ctypes.create_string_buffer(n5)
    assert L.bitnet_grouped_plan_linear(ctypes.cast(arr5, ctypes.c_void_p), 2,
                                        ctypes.cast(buf5, ctypes.c_void_p), n5) == OK
    hdr5 = (ctypes.c_uint32 * 8).from_buffer_copy(buf5.raw[:32])
    assert hdr5[7] == 1 and hdr5[5] == 256 and hdr5[3] == 2 + 1
    assert hdr[7] == 0


def test_python_binding_fails_loudly_without_gpu_tensors():
    import torch
    q = torch.zeros((1, 64), dtype=torch.int8)
    with pytest.raises(ValueError):
        tw.bitnet_linear(q, torch.zeros(1), torch.zeros((4, 16), dtype=torch.uint8),
                         torch.zeros(1), torch.zeros((1, 4)))


def test_grouped_plan_builders_reject_host_tensors():
    """The plan builders check every tensor before anything reaches the C planner."""
    import torch
    q = torch.zeros((1, 64), dtype=torch.int8)
    s = torch.zeros(1)
    p = torch.zeros((4, 16), dtype=torch.uint8)
    y = torch.zeros((1, 4))
    with pytest.raises(ValueError):
        tw.bitnet_grouped_plan_linear([(q, s, p, s, y, None)])
    with pytest.raises(ValueError):
        tw.bitnet_grouped_plan_quant([(torch.zeros((1, 64), dtype=torch.bfloat16), q, s)])
    with pytest.raises(ValueError):
        tw.bitnet_grouped_plan_fused([(torch.zeros((1, 64), dtype=torch.bfloat16), p, s, y, None, None, None)])


def test_fused_plan_checks(L):
    F = tw._FusedDesc
    a16 = 4096
    good = F(a16, a16, a16, a16, 0, 0, 0, 1, 300, 2560)
    arr = (F * 1)(good)
    n = L.bitnet_grouped_plan_fused_bytes(1, ctypes.cast(arr, ctypes.c_void_p))
    buf = ctypes.create_string_buffer(n)
    assert L.bitnet_grouped_plan_fused(ctypes.cast(arr, ctypes.c_void_p), 1, ctypes.cast(buf, ctypes.c_void_p), n) == OK
    hdr = (ctypes.c_uint32 * 8).from_buffer_copy(buf.raw[:32])
    assert hdr[1] == 3 and hdr[3] == (300 + 127) // 128 and hdr[5] == 128
    assert L.bitnet_grouped_plan_fused(ctypes.cast(arr, ctypes.c_void_p), 1, ctypes.cast(buf, ctypes.c_void_p), n - 1) == ARG
    bad = [
        (F(a16, a16, a16, a16, 0, 0, 0, 2, 300, 2560), SHAPE),      # one token per problem
        (F(a16, a16, a16, a16, 0, 0, 0, 1, 300, 52224 + 64), SHAPE),  # q must fit one LDS segment
        (F(a16 + 2, a16, a16, a16, 0, 0, 0, 1, 300, 2560), ALIGN),    # x 16-byte aligned
        (F(a16, a16, a16, a16, 0, a16 + 8, 0, 1, 300, 2560), ALIGN),  # q 16-byte aligned
        (F(a16, a16, a16, a16, 0, 0, 0, 1, 300, 2528), ALIGN),        # K % 64
        (F(0, a16, a16, a16, 0, 0, 0, 1, 300, 2560), NULL),
    ]
    for d, want in bad:
        one = (F * 1)(d)
        assert L.bitnet_grouped_plan_fused(ctypes.cast(one, ctypes.c_void_p), 1, ctypes.cast(buf, ctypes.c_void_p),
                                           n) == want, (d.M, d.K, want)
    # a fused plan is not a linear or quant plan
    dev = ctypes.c_void_p(4096)
    assert L.bitnet_linear_grouped(ctypes.cast(buf, ctypes.c_void_p), dev, None) == ARG
    assert L.bitnet_quant_act_grouped(ctypes.cast(buf, ctypes.c_void_p), dev, None) == ARG


def test_rmsnorm_quant_rejects_bad_arguments(L):
    p = ctypes.c_void_p(256)  # never dereferenced: every call below fails its checks
    z = None
    f = ctypes.c_float
    assert L.bitnet_rmsnorm_quant_act(p, z, f(1e-6), 1, 64, p, p, z) == NULL
    assert L.bitnet_rmsnorm_quant_act(p, p, f(1e-6), 1, 60, p, p, z) == SHAPE    # K % 8
    assert L.bitnet_rmsnorm_quant_act(ctypes.c_void_p(264), p, f(1e-6), 1, 64, p, p, z) == ALIGN
    assert L.bitnet_rmsnorm_quant_act(p, ctypes.c_void_p(260), f(1e-6), 1, 64, p, p, z) == ALIGN
    assert L.bitnet_rmsnorm_quant_act(p, p, f(-1.0), 1, 64, p, p, z) == ARG
    assert L.bitnet_rmsnorm_quant_act(p, p, f(float("nan")), 1, 64, p, p, z) == ARG
    assert L.bitnet_rmsnorm_quant_act(z, z, f(0.0), 0, 64, z, z, z) == OK


def test_fused_plan_norm_checks_and_variant(L):
    F = tw._FusedDesc
    a16 = 4096
    n = ctypes.c_float
    good = F(a16, a16, a16, a16, 0, 0, 0, 1, 300, 2560, a16, n(1e-6))
    arr = (F * 2)(good, F(a16, a16, a16, a16, 0, 0, 0, 1, 300, 2560, 0, n(0.0)))
    nb = L.bitnet_grouped_plan_fused_bytes(2, arr)
    buf = ctypes.create_string_buffer(nb)
    assert L.bitnet_grouped_plan_fused(arr, 2, buf, nb) == OK
    hdr = (ctypes.c_uint32 * 8).from_buffer_copy(buf.raw[:32])
    assert hdr[1] == 3 and hdr[7] == 1          # fused plan, variant with RMSNorm
    arr1 = (F * 1)(F(a16, a16, a16, a16, 0, 0, 0, 1, 300, 2560, 0, n(0.0)))
    nb1 = L.bitnet_grouped_plan_fused_bytes(1, arr1)
    buf1 = ctypes.create_string_buffer(nb1)
    assert L.bitnet_grouped_plan_fused(arr1, 1, buf1, nb1) == OK
    assert (ctypes.c_uint32 * 8).from_buffer_copy(buf1.raw[:32])[7] == 0
    for d, want in ((F(a16, a16, a16, a16, 0, 0, 0, 1, 300, 2560, a16 + 4, n(1e-6)), ALIGN),
                    (F(a16, a16, a16, a16, 0, 0, 0, 1, 300, 2560, a16, n(-1.0)), ARG)):
        one = (F * 1)(d)
        assert L.bitnet_grouped_plan_fused(one, 1, buf, nb) == want


def test_swiglu_quant_rejects_bad_arguments(L):
    p = ctypes.c_void_p(256)  # never dereferenced: every call below fails its checks
    z = None
    assert L.bitnet_swiglu_quant_act(p, z, 1, 64, p, p, z) == NULL
    assert L.bitnet_swiglu_quant_act(p, p, 1, 60, p, p, z) == SHAPE     # K % 8
    assert L.bitnet_swiglu_quant_act(ctypes.c_void_p(264), p, 1, 64, p, p, z) == ALIGN
    assert L.bitnet_swiglu_quant_act(p, ctypes.c_void_p(260), 1, 64, p, p, z) == ALIGN
    assert L.bitnet_swiglu_quant_act(p, p, 1, 64, ctypes.c_void_p(264), p, z) == ALIGN
    assert L.bitnet_swiglu_quant_act(p, p, -1, 64, p, p, z) == SHAPE
    assert L.bitnet_swiglu_quant_act(z, z, 0, 64, z, z, z) == OK


def test_fused_plan_swiglu_checks_and_variant(L):
    F = tw._FusedDesc
    a16 = 4096
    n = ctypes.c_float

    def plan(*descs):
        arr = (F * len(descs))(*descs)
        nb = L.bitnet_grouped_plan_fused_bytes(len(descs), arr)
        buf = ctypes.create_string_buffer(nb)
        assert L.bitnet_grouped_plan_fused(arr, len(descs), buf, nb) == OK
        return (ctypes.c_uint32 * 8).from_buffer_copy(buf.raw[:32])

    plain = F(a16, a16, a16, a16, 0, 0, 0, 1, 300, 2560, 0, n(0.0), 0, 0, 0)
    norm = F(a16, a16, a16, a16, 0, 0, 0, 1, 300, 2560, a16, n(1e-6), 0, 0, 0)
    f32 = F(0, a16, a16, a16, 0, 0, 0, 1, 2560, 6912, 0, n(0.0), a16, 0, 0)
    pair = F(a16, a16, a16, a16, 0, 0, 0, 1, 6912, 2560, a16, n(1e-6), 0, a16, a16)
    assert plan(plain)[7] == 0 and plan(norm)[7] == 1 and plan(f32)[7] == 2 and plan(pair)[7] == 3
    assert plan(plain, f32)[7] == 2 and plan(norm, plain, f32)[7] == 3
    # blocks: R rows per block, R / 2 for a pair (each row of both matrices)
    R = plan(f32)[5]
    assert plan(f32)[3] == -(-2560 // R) and plan(pair)[3] == -(-6912 // (R // 2))
    assert plan(pair, f32)[3] == -(-6912 // (R // 2)) - (-2560 // R)
    buf = ctypes.create_string_buffer(4096)
    for d, want in ((F(a16, a16, a16, a16, 0, 0, 0, 1, 300, 6912, 0, n(0.0), a16, 0, 0), ARG),   # x and x_f32
                    (F(0, a16, a16, a16, 0, 0, 0, 1, 300, 6912, a16, n(0.0), a16, 0, 0), ARG),   # x_f32 and a norm
                    (F(0, a16, a16, a16, 0, 0, 0, 1, 300, 6912, 0, n(0.0), a16 + 4, 0, 0), ALIGN),
                    (F(a16, a16, a16, a16, 0, 0, 0, 1, 300, 2560, 0, n(0.0), 0, a16, 0), NULL),  # s_w_up missing
                    (F(a16, a16, a16, a16, 0, 0, 0, 1, 300, 2560, 0, n(0.0), 0, 0, a16), NULL),  # packed_up missing
                    (F(a16, a16, a16, a16, a16, 0, 0, 1, 300, 2560, 0, n(0.0), 0, a16, a16), ARG),  # pair with acc
                    (F(0, a16, a16, a16, 0, 0, 0, 1, 300, 2560, 0, n(0.0), a16, a16, a16), ARG),  # pair on fp32 x
                    (F(a16, a16, a16, a16, 0, 0, 0, 1, 300, 2560, 0, n(0.0), 0, a16 + 8, a16), ALIGN),
                    (F(a16, a16, a16, a16, 0, 0, 0, 1, 300, 2560, 0, n(0.0), 0, a16, a16 + 2), ALIGN)):
        one = (F * 1)(d)
        assert L.bitnet_grouped_plan_fused(one, 1, buf, 4096) == want


def test_bit_encodings_reject_bad_arguments(L):
    p = ctypes.c_void_p(4096)  # never dereferenced: every call below fails its checks
    z = None
    ws = ctypes.c_size_t(1 << 20)
    assert L.bitnet_pack_weights_binary(p, 4, 48, p, p, p, ws, z) == SHAPE        # K % 32
    assert L.bitnet_pack_weights_binary(p, 4, 64, p, z, p, ws, z) == NULL
    assert L.bitnet_pack_weights_binary(ctypes.c_void_p(4100), 4, 64, p, p, p, ws, z) == ALIGN
    assert L.bitnet_pack_weights_binary(p, 4, 64, p, p, p, ctypes.c_size_t(8), z) == ARG  # workspace
    assert L.bitnet_pack_bitplanes(p, 4, 48, p, z) == SHAPE
    assert L.bitnet_pack_bitplanes(ctypes.c_void_p(4100), 4, 64, p, z) == ALIGN
    assert L.bitnet_pack_bitplanes(z, 4, 64, p, z) == NULL
    assert L.bitnet_pack_bitplanes(z, 0, 64, z, z) == OK
    lb = L.bitnet_linear_bits
    assert lb(p, p, p, 3, p, 1, 8, 128, p, z, 0, z) == ARG                        # format
    assert lb(p, p, p, 1, p, 1, 8, 128, p, z, 5, z) == ARG                        # kernel id
    assert lb(p, p, p, 1, p, 2, 8, 96, p, z, 4, z) == ARG                         # MFMA kernel, binary: K % 64
    assert lb(p, p, p, 2, p, 2, 8, 96, p, z, 4, z) == ARG                         # MFMA kernel: K % 64
    assert lb(p, p, p, 2, p, 16 * 65536, 8, 128, p, z, 4, z) == ARG               # MFMA kernel: token tiles
    assert lb(p, p, ctypes.c_void_p(4104), 2, p, 2, 8, 128, p, z, 4, z) == ARG    # MFMA kernel: alignment
    assert lb(p, p, p, 1, p, 2, 8, 96, p, z, 3, z) == ARG                         # multi-token binary: K % 128
    assert lb(p, p, p, 2, p, 2, 8, 96, p, z, 3, z) == ARG                         # multi-token bitplanes: K % 64
    assert lb(p, p, p, 1, p, 65536, 8, 128, p, z, 3, z) == ARG                    # token tiles on the grid's y
    assert lb(ctypes.c_void_p(4097), p, p, 1, p, 2, 8, 128, p, z, 3, z) == ARG    # alignment
    assert lb(p, p, p, 1, p, 1, 8, 100, p, z, 0, z) == SHAPE                      # K % 32
    assert lb(p, p, z, 1, p, 1, 8, 128, p, z, 0, z) == NULL
    assert lb(p, p, p, 1, p, 2, 8, 128, p, z, 2, z) == ARG                        # GEMV: M == 1
    assert lb(p, p, p, 1, p, 1, 8, 96, p, z, 2, z) == ARG                         # binary GEMV: K % 128
    assert lb(p, p, p, 2, p, 1, 8, 96, p, z, 2, z) == ARG                         # bitplanes GEMV: K % 64
    assert lb(p, p, p, 1, p, 1, 8, 57344 + 128, p, z, 2, z) == ARG                # LDS limit
    assert lb(ctypes.c_void_p(4097), p, p, 1, p, 1, 8, 128, p, z, 2, z) == ARG    # alignment
    assert lb(p, p, p, 1, p, 0, 8, 128, p, z, 0, z) == OK


def test_fused_plan_bitplanes(L):
    F = tw._FusedDesc
    a16 = 4096
    n = ctypes.c_float
    arr = (F * 2)(F(a16, a16, a16, a16, 0, 0, 0, 1, 2560, 6912, 0, n(0.0), 0, 0, 0, 2),
                  F(a16, a16, a16, a16, 0, 0, 0, 1, 300, 2560, 0, n(0.0), 0, 0, 0, 2))
    nb = L.bitnet_grouped_plan_fused_bytes(2, arr)
    buf = ctypes.create_string_buffer(nb)
    assert L.bitnet_grouped_plan_fused(arr, 2, buf, nb) == OK
    hdr = (ctypes.c_uint32 * 8).from_buffer_copy(buf.raw[:32])
    assert hdr[7] == 4 and hdr[3] == -(-2560 // hdr[5]) - (-300 // hdr[5])
    bad = [
        (F(a16, a16, a16, a16, 0, 0, 0, 1, 300, 2560, 0, n(0.0), 0, 0, 0, 1), ARG),          # binary: not here
        (F(a16, a16, a16, a16, 0, 0, 0, 1, 300, 2560, a16, n(1e-6), 0, 0, 0, 2), ARG),       # no norm
        (F(0, a16, a16, a16, 0, 0, 0, 1, 300, 2560, 0, n(0.0), a16, 0, 0, 2), ARG),          # no fp32 row
        (F(a16, a16, a16, a16, 0, 0, 0, 1, 300, 2560, 0, n(0.0), 0, a16, a16, 2), ARG),      # no pair
        (F(a16, a16, a16, a16, 0, 0, 0, 1, 300, 51584 + 64, 0, n(0.0), 0, 0, 0, 2), SHAPE),  # LDS limit
    ]
    for d, want in bad:
        one = (F * 1)(d)
        assert L.bitnet_grouped_plan_fused(one, 1, buf, nb) == want
    mixed = (F * 2)(F(a16, a16, a16, a16, 0, 0, 0, 1, 300, 2560, 0, n(0.0), 0, 0, 0, 2),
                    F(a16, a16, a16, a16, 0, 0, 0, 1, 300, 2560, 0, n(0.0), 0, 0, 0, 0))
    assert L.bitnet_grouped_plan_fused(mixed, 2, buf, nb) == ARG


def test_linear_plan_weight_groups(L):
    D = tw._LinearDesc
    a16 = 4096
    arr = (D * 2)(D(a16, a16, a16, a16, a16, 0, 1, 300, 2560, 0), D(a16, a16, a16, a16, a16, 0, 3, 200, 2560, 128))
    nb = L.bitnet_grouped_plan_bytes(2, 1, arr)
    buf = ctypes.create_string_buffer(nb)
    assert L.bitnet_grouped_plan_linear(arr, 2, buf, nb) == OK
    hdr = (ctypes.c_uint32 * 8).from_buffer_copy(buf.raw[:32])
    assert hdr[7] == 4                          # MFMA decode kernel with its group-wise path
    R = hdr[5]                                  # one block per R rows, all tokens at once
    assert R == 256 and hdr[3] == -(-300 // R) + -(-200 // R)
    one = (D * 1)(D(a16, a16, a16, a16, a16, 0, 1, 200, 2560, 128))    # every M = 1: the GEMV, one token each
    nb1 = L.bitnet_grouped_plan_bytes(1, 1, one)
    assert L.bitnet_grouped_plan_linear(one, 1, buf, nb1) == OK
    hdr = (ctypes.c_uint32 * 8).from_buffer_copy(buf.raw[:32])
    R1 = hdr[5]
    assert hdr[7] == 2 and R1 > 0 and hdr[3] == -(-200 // R1)
    for w_group in (96, 32, -64):               # not dividing K / not a multiple of 64
        bad = (D * 1)(D(a16, a16, a16, a16, a16, 0, 1, 300, 2560, w_group))
        assert L.bitnet_grouped_plan_linear(bad, 1, buf, nb) == SHAPE
    ok = (D * 1)(D(a16, a16, a16, a16, a16, 0, 2, 300, 2560, 2560))     # per channel: MFMA variant stays
    assert L.bitnet_grouped_plan_linear(ok, 1, buf, nb) == OK
    assert (ctypes.c_uint32 * 8).from_buffer_copy(buf.raw[:32])[7] == 1
    # header flags (the last 8 header bytes): bit 0 set only when a group-wise problem
    # asks for its int32 acc (the several-token kernel then keeps the integer sums)
    assert L.bitnet_grouped_plan_linear(arr, 2, buf, nb) == OK
    assert ctypes.c_uint64.from_buffer_copy(buf.raw[56:64]).value == 0
    acc_plain = (D * 2)(D(a16, a16, a16, a16, a16, a16, 1, 300, 2560, 0), D(a16, a16, a16, a16, a16, 0, 3, 200, 2560, 128))
    assert L.bitnet_grouped_plan_linear(acc_plain, 2, buf, nb) == OK
    assert ctypes.c_uint64.from_buffer_copy(buf.raw[56:64]).value == 0
    acc_group = (D * 2)(D(a16, a16, a16, a16, a16, 0, 1, 300, 2560, 0), D(a16, a16, a16, a16, a16, a16, 3, 200, 2560, 128))
    assert L.bitnet_grouped_plan_linear(acc_group, 2, buf, nb) == OK
    assert ctypes.c_uint64.from_buffer_copy(buf.raw[56:64]).value == 1


def test_linear_plan_lds_covers_every_descriptor(L):
    """The plan's dynamic LDS size covers each descriptor's own staging: a plain
    K = 51200 row stages all 800 chunks at 20 dwords (64000 bytes) in one segment,
    while group-wise descriptors keep 21 dwords per chunk and split such a K."""
    D = tw._LinearDesc
    a16 = 4096
    mixed = (D * 2)(D(a16, a16, a16, a16, a16, 0, 1, 64, 51200, 0), D(a16, a16, a16, a16, a16, 0, 1, 64, 2560, 128))
    nb = L.bitnet_grouped_plan_bytes(2, 1, mixed)
    buf = ctypes.create_string_buffer(nb)
    assert L.bitnet_grouped_plan_linear(mixed, 2, buf, nb) == OK
    hdr = (ctypes.c_uint32 * 8).from_buffer_copy(buf.raw[:32])
    assert hdr[7] == 2 and hdr[6] >= 800 * 20 * 4
    alone = (D * 1)(D(a16, a16, a16, a16, a16, 0, 1, 64, 51200, 128))
    assert L.bitnet_grouped_plan_linear(alone, 1, buf, nb) == OK
    hdr = (ctypes.c_uint32 * 8).from_buffer_copy(buf.raw[:32])
    assert 0 < hdr[6] <= 64 * 1024


def test_plan_output_options_checks(L):
    """Bias and bf16 y per descriptor: dtype and alignment checks, and the forms that
    take neither (a gate / up pair takes no bias; bitplane plans take fp32 y, no bias)."""
    D, F = tw._LinearDesc, tw._FusedDesc
    a16 = 4096
    n = ctypes.c_float
    buf = ctypes.create_string_buffer(8192)

    def lin(**kw):
        d = D(a16, a16, a16, a16, a16, 0, 1, 100, 2560, 0)
        for k, v in kw.items():
            setattr(d, k, v)
        return L.bitnet_grouped_plan_linear((D * 1)(d), 1, buf, 8192)

    assert lin() == OK
    assert lin(bias=a16, y_dtype=1) == OK
    assert lin(y_dtype=2) == ARG
    assert lin(y=a16 + 2) == ALIGN                 # fp32 y: 4-byte aligned
    assert lin(y=a16 + 2, y_dtype=1) == OK         # bf16 y: 2-byte aligned
    assert lin(bias=a16 + 2) == ALIGN

    def fused(**kw):
        d = F(a16, a16, a16, a16, 0, 0, 0, 1, 300, 2560, 0, n(0.0), 0, 0, 0, 0)
        for k, v in kw.items():
            setattr(d, k, v)
        return L.bitnet_grouped_plan_fused((F * 1)(d), 1, buf, 8192)

    assert fused() == OK
    assert fused(bias=a16, y_dtype=1) == OK
    assert fused(y_dtype=3) == ARG
    assert fused(y=a16 + 1, y_dtype=1) == ALIGN
    assert fused(bias=a16 + 1) == ALIGN
    assert fused(packed_up=a16, s_w_up=a16, y_dtype=1) == OK
    assert fused(packed_up=a16, s_w_up=a16, bias=a16) == ARG      # no bias on a pair
    assert fused(weight_fmt=2, bias=a16) == ARG                   # bitplanes: no bias
    assert fused(weight_fmt=2, y_dtype=1) == ARG                  # bitplanes: fp32 y


def test_plan_builders_check_output_options():
    import torch
    q = torch.zeros((1, 64), dtype=torch.int8)
    with pytest.raises(ValueError):
        # a host tensor is refused before anything else
        tw.bitnet_grouped_plan_linear([(q, torch.zeros(1), torch.zeros((4, 16), dtype=torch.uint8), torch.zeros(1),
                                        torch.zeros((1, 4), dtype=torch.float16), None)])
