"""GPU parity: every entry point of the HIP library (through the C ABI and its
Python binding) against the CPU oracle, element by element, on the same seeded
inputs.  Integer and byte outputs (packed bytes, s_w, q, s_x, acc) must be
identical, and so must fp32 y wherever the row has one weight scale (per tensor or
per output channel): the library and the oracle both form y = acc * c_m (+ bias)
in float64 with c_m = (s_x s_w) / 127 and round once to fp32.  The options whose
sums run in another order than the oracle's are held to derived bounds:
group-wise weight scales (float64 sums over groups) and RMSNorm rows (s_x from a
float64 sum of squares, one fp32 unit from the oracle's at most).

Small and medium shapes are compared in full (several tiles plus ragged tails);
the full-size workloads (the 2.4B decode step, the M = 2048 prefill shapes and
the 100B-scale FFN shapes) are compared on sampled rows and columns, in the
launch configuration the bench uses.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import workloads as W
import ternary_weight_token_amd as tw

pytestmark = pytest.mark.gpu

REL = 2.0 ** -23
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    tw.lib()  # raises if the HIP library is missing: no fallback exists
    oracle.set_threads(min(16, max(1, len(__import__("os").sched_getaffinity(0)))))


# ----------------------------------------------------------------- helpers

def bits_np(x_bf16_cpu: torch.Tensor) -> np.ndarray:
    return synth.bf16_bits(x_bf16_cpu.contiguous()).numpy().view(np.uint16)


def assert_y(y_gpu: np.ndarray, y_ref: np.ndarray):
    """fp32 outputs bit for bit (the same float64 factor and product, one rounding)."""
    a = np.ascontiguousarray(y_gpu, dtype=np.float32).view(np.uint32)
    b = np.ascontiguousarray(y_ref, dtype=np.float32).view(np.uint32)
    bad = a != b
    assert not bad.any(), f"{bad.sum()} fp32 outputs differ from the oracle; first at {np.argwhere(bad)[0]}"


def assert_y_within(y_gpu: np.ndarray, y_ref: np.ndarray, rel: float, slack=0.0):
    d = np.abs(y_gpu.astype(np.float64) - y_ref.astype(np.float64))
    bad = d > rel * np.abs(y_ref.astype(np.float64)) + slack
    assert not bad.any(), f"{bad.sum()} outputs outside the bound; first at {np.argwhere(bad)[0]}"


def assert_bf16(y_bits: np.ndarray, y_ref32: np.ndarray):
    """bf16 outputs: the oracle's fp32 y rounded to nearest even, bit for bit."""
    want = oracle.to_bf16(np.ascontiguousarray(y_ref32, dtype=np.float32))
    bad = np.asarray(y_bits).view(np.uint16) != want
    assert not bad.any(), f"{bad.sum()} bf16 outputs differ from the oracle; first at {np.argwhere(bad)[0]}"


def gpu_quant(x_cpu):
    q, s = tw.quant_act(x_cpu.to(DEV))
    return q.cpu().numpy(), s.cpu().numpy()


def gpu_linear(q_np, s_np, packed_np, s_w, want_acc=True, kernel=0):
    """kernel 0: bitnet_linear's own choice; else forced (1 GEMV, 2 GEMM, 4 MFMA decode)."""
    q = torch.from_numpy(q_np).to(DEV)
    s = torch.from_numpy(s_np).to(DEV)
    p = torch.from_numpy(packed_np).to(DEV)
    sw = torch.tensor([s_w], dtype=torch.float32, device=DEV)
    if kernel == 0:
        y, acc = tw.linear(q, s, p, sw, want_acc=True)
    else:
        y = torch.empty((q.shape[0], p.shape[0]), dtype=torch.float32, device=DEV)
        acc = torch.empty((q.shape[0], p.shape[0]), dtype=torch.int32, device=DEV)
        tw.bitnet_linear_select(q, s, p, sw, y, acc, kernel)
    return y.cpu().numpy(), acc.cpu().numpy()


def check_linear(q_np, s_np, packed_np, s_w, kernels=(0,)):
    acc_ref, y_ref = oracle.linear(q_np, s_np, packed_np, s_w)
    for kern in kernels:
        y, acc = gpu_linear(q_np, s_np, packed_np, s_w, kernel=kern)
        assert np.array_equal(acc, acc_ref), kern
        assert_y(y, y_ref)
    return acc, y


def quantized_inputs(key, M, K, **kw):
    x = synth.activations(key, M, K, **kw)
    q, s = oracle.quant_act(bits_np(x))
    return x, q, s


# ----------------------------------------------------------------- quant_act

@pytest.mark.parametrize("M,K,kw", [
    (1, 2560, dict(outlier_frac=0.001)),
    (1, 6912, {}),
    (3, 2560, dict(outlier_frac=0.01)),
    (17, 64, {}),
    (64, 2560, dict(outlier_frac=0.001)),
    (2048, 6912, dict(row_scale=(0.1, 10.0))),
    (5, 68, {}),        # K % 8 != 0: scalar path
    (2, 4, {}),         # smallest K
    (1, 28672, {}),
])
def test_quant_act_parity(M, K, kw):
    x = synth.activations(synth.stream_key(100, M, K), M, K, **kw)
    q_ref, s_ref = oracle.quant_act(bits_np(x))
    q, s = gpu_quant(x)
    assert np.array_equal(q, q_ref)
    assert np.array_equal(s, s_ref)


def test_quant_act_grouped_rows():
    """The grouped quantization plan (one wavefront per row): rows of 8 .. 16392 values
    (up to two passes over a row), an all-zero row, outliers, several tokens per
    problem and problems of different K in one launch; q and s_x bit for bit."""
    shapes = [(1, 8), (3, 64), (8, 2560), (2, 6912), (5, 8192), (1, 8200), (4, 16392), (9, 640)]
    probs, refs = [], []
    for i, (M, K) in enumerate(shapes):
        x = synth.activations(synth.stream_key(104, i, M, K), M, K, outlier_frac=0.002)
        if i == 2:
            x[1].zero_()
        refs.append(oracle.quant_act(bits_np(x)))
        xd = x.to(DEV)
        probs.append((xd, torch.full((M, K), 99, dtype=torch.int8, device=DEV),
                      torch.full((M,), -1.0, dtype=torch.float32, device=DEV)))
    plan = tw.bitnet_grouped_plan_quant(probs)
    for _ in range(2):
        plan.launch()
        torch.cuda.synchronize()
        for (q_ref, s_ref), (xd, q, s) in zip(refs, probs):
            assert np.array_equal(q.cpu().numpy(), q_ref)
            assert np.array_equal(s.cpu().numpy(), s_ref)


@pytest.mark.parametrize("fused", [False, True])
def test_quant_act_exhaustive_bf16(fused):
    """Every finite bf16 value x with |x| <= s, for scales s across the whole range
    (subnormal, tiny, ordinary, large), quantized on the GPU (bitnet_quant_act, or
    inside the fused launch) against the oracle's exact rounding of 127 x / s."""
    pos = np.arange(0, 0x7F80, dtype=np.uint32)              # +0 .. largest finite
    vals = (pos << 16).view(np.float32)
    scales = [np.uint16(b) for b in (0x0001, 0x0080, 0x0D80, 0x3A00, 0x3F80, 0x4040, 0x42FE, 0x4B00, 0x5F00, 0x7A00)]
    for sb in scales:
        s = np.array([np.uint32(sb) << 16], dtype=np.uint32).view(np.float32)[0]
        xb = pos[vals <= s].astype(np.uint16)
        row = np.concatenate([xb, xb | np.uint16(0x8000)])          # both signs, contains s itself
        K = 52224 if fused else -(-len(row) // 64) * 64
        reps = -(-K // len(row))
        row = np.tile(row, reps)[:K] if len(row) < K else row[:K]
        if not np.any((row & 0x7FFF) == sb):                     # keep the row max at s
            row[0] = sb
        x_bits = row.reshape(1, K).view(np.uint16)
        q_ref, s_ref = oracle.quant_act(x_bits)
        x = torch.from_numpy(x_bits.view(np.int16).copy()).view(torch.bfloat16).to(DEV)
        if not fused:
            q, sx = tw.quant_act(x)
        else:
            packed = torch.full((64, K // 4), 0x55, dtype=torch.uint8, device=DEV)
            y = torch.empty((1, 64), dtype=torch.float32, device=DEV)
            q = torch.empty((1, K), dtype=torch.int8, device=DEV)
            sx = torch.empty(1, dtype=torch.float32, device=DEV)
            tw.bitnet_grouped_plan_fused([(x, packed, torch.ones(1, device=DEV), y, None, q, sx)]).launch()
        torch.cuda.synchronize()
        assert np.array_equal(sx.cpu().numpy(), s_ref), hex(int(sb))
        assert np.array_equal(q.cpu().numpy(), q_ref), hex(int(sb))


def test_quant_act_zero_rows_and_unaligned():
    x = synth.activations(synth.stream_key(101), 6, 512)
    x[2] = 0
    x[5] = -0.0
    q_ref, s_ref = oracle.quant_act(bits_np(x))
    q, s = gpu_quant(x)
    assert np.array_equal(q, q_ref) and np.array_equal(s, s_ref)
    assert s[2] == 0 and np.all(q[2] == 0)
    # x starting 2 bytes past a 16-byte boundary takes the general path
    big = torch.zeros(6 * 512 + 1, dtype=torch.bfloat16, device=DEV)
    big[1:] = x.reshape(-1).to(DEV)
    xv = big[1:].view(6, 512)
    q2 = torch.empty((6, 512), dtype=torch.int8, device=DEV)
    s2 = torch.empty(6, dtype=torch.float32, device=DEV)
    tw.bitnet_quant_act(xv, q2, s2)
    assert np.array_equal(q2.cpu().numpy(), q_ref) and np.array_equal(s2.cpu().numpy(), s_ref)


# ----------------------------------------------------------------- pack

@pytest.mark.parametrize("N,K,kind", [
    (2560, 2560, "normal"), (37, 68, "normal"), (5, 4, "normal"), (64, 6912, "normal"),
    (40, 256, "zero"), (256, 2560, "d0.3"), (256, 2560, "d0.5"), (256, 2560, "d0.7"),
])
def test_pack_parity(N, K, kind):
    key = synth.stream_key(200, N, K)
    if kind == "normal":
        w = synth.latent_weights(key, N, K, 0.02)
    elif kind == "zero":
        w = torch.zeros((N, K), dtype=torch.float32)
    else:
        w = synth.density_weights(key, N, K, float(kind[1:]))
    p_ref, s_ref = oracle.pack(w.numpy(), 1e-5)
    p, s = tw.pack_weights(w.to(DEV), 1e-5)
    assert s.item() == s_ref
    assert np.array_equal(p.cpu().numpy(), p_ref)


def test_pack_eps_zero_ties():
    w = torch.tensor([[2.0, 0.5, -0.5, 1.0] * 16], dtype=torch.float32)
    p_ref, s_ref = oracle.pack(w.numpy(), 0.0)
    p, s = tw.pack_weights(w.to(DEV), 0.0)
    assert s.item() == s_ref and np.array_equal(p.cpu().numpy(), p_ref)
    assert np.all(p.cpu().numpy() == 0x96)


# ----------------------------------------------------------------- linear

@pytest.mark.parametrize("M", list(range(1, 17)))
def test_gemv_parity_all_m(M):
    # N = 300 is not a multiple of the row block; K = 2624 gives 41 chunks of
    # 64 weights per row, not a multiple of the 8 lanes that walk a row.
    N, K = 300, 2624
    key = synth.stream_key(300, M)
    x, q, s = quantized_inputs(key, M, K, outlier_frac=0.001)
    packed = synth.random_bytes(synth.stream_key(key, 1), N * K // 4).numpy().reshape(N, K // 4)
    check_linear(q, s, packed, np.float32(0.0113), kernels=(0, 1))


@pytest.mark.parametrize("M,N,K", [(1, 64, 6912), (1, 33, 28672), (4, 640, 2560), (16, 1000, 8192),
                                   (1, 1, 64), (2, 7, 128),
                                   (1, 16400, 2560), (1, 16384, 8192)])   # tall: 4 rows per octet
def test_gemv_parity_shapes(M, N, K):
    key = synth.stream_key(301, M, N, K)
    x, q, s = quantized_inputs(key, M, K)
    w = synth.latent_weights(synth.stream_key(key, 1), N, K, 0.02)
    packed, s_w = oracle.pack(w.numpy())
    check_linear(q, s, packed, s_w, kernels=(0, 1))


@pytest.mark.parametrize("M,N,K", [(1, 300, 2624), (2, 70, 26176), (3, 200, 64), (5, 33, 8192),
                                   (8, 1000, 6912), (11, 129, 2560), (16, 65, 28672), (17, 97, 640),
                                   (40, 300, 1024)])
def test_mfma_decode_kernel(M, N, K):
    """The MFMA decode kernel, forced: ragged N, K slices with ragged tails, M below
    and above one 16-token tile."""
    key = synth.stream_key(308, M, N, K)
    x, q, s = quantized_inputs(key, M, K, row_scale=(0.1, 10.0))
    packed = synth.random_bytes(synth.stream_key(key, 1), N * K // 4).numpy().reshape(N, K // 4)
    acc_ref, y_ref = oracle.linear(q, s, packed, np.float32(0.0117))
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    tw.bitnet_linear_select(torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV),
                            torch.from_numpy(packed).to(DEV), torch.tensor([0.0117], device=DEV),
                            y, acc, 4)
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert_y(y.cpu().numpy(), y_ref)


@pytest.mark.parametrize("with_outputs", [True, False])
def test_fused_quant_linear_grouped(with_outputs):
    """One fused grouped launch (quantization inside the GEMV workgroups) against the
    oracle's quant_act + linear, problem by problem: ragged N, K from one chunk to the
    longest single-segment K, an all-zero row, outliers, rows of every scale."""
    shapes = [(300, 2560, {}), (129, 52224, {"outlier_frac": 0.001}), (64, 64, {}), (97, 6912, {"row_scale": (1e-3, 1e-3)}),
              (700, 640, {"outlier_frac": 0.01}), (33, 2560, "zero")]
    probs, refs = [], []
    for i, (N, K, kw) in enumerate(shapes):
        key = synth.stream_key(309, i)
        x = torch.zeros((1, K), dtype=torch.bfloat16) if kw == "zero" else synth.activations(key, 1, K, **kw)
        packed = synth.random_bytes(synth.stream_key(key, 1), N * K // 4).numpy().reshape(N, K // 4)
        s_w = np.float32(0.0093 * (i + 1))
        q_ref, sx_ref = oracle.quant_act(bits_np(x))
        acc_ref, y_ref = oracle.linear(q_ref, sx_ref, packed, s_w)
        refs.append((q_ref, sx_ref, acc_ref, y_ref))
        y = torch.full((1, N), float("nan"), dtype=torch.float32, device=DEV)
        acc = torch.empty((1, N), dtype=torch.int32, device=DEV)
        q = torch.full((1, K), 99, dtype=torch.int8, device=DEV) if with_outputs else None
        sx = torch.full((1,), -1.0, dtype=torch.float32, device=DEV) if with_outputs else None
        probs.append((x.to(DEV), torch.from_numpy(packed).to(DEV), torch.tensor([s_w], device=DEV), y, acc, q, sx))
    plan = tw.bitnet_grouped_plan_fused(probs)
    for _ in range(2):
        for pr in probs:
            pr[3].fill_(float("nan"))
            pr[4].fill_(-1)
        plan.launch()
        torch.cuda.synchronize()
        for (q_ref, sx_ref, acc_ref, y_ref), pr in zip(refs, probs):
            assert np.array_equal(pr[4].cpu().numpy(), acc_ref)
            assert_y(pr[3].cpu().numpy(), y_ref)
            if with_outputs:
                assert np.array_equal(pr[5].cpu().numpy(), q_ref)
                assert np.array_equal(pr[6].cpu().numpy(), sx_ref)


# ----------------------------------------------------------------- group-wise weight scales

@pytest.mark.parametrize("N,K,G", [(300, 2560, 128), (33, 6912, 6912), (70, 640, 64), (5, 68, 4), (129, 512, 512)])
def test_pack_grouped_parity(N, K, G):
    key = synth.stream_key(330, N, K, G)
    w = synth.latent_weights(key, N, K, 0.02)
    w[:, :G] *= 4.0
    p_ref, s_ref = oracle.pack_grouped(w.numpy(), G, 1e-5)
    p, sw = tw.pack_weights_grouped(w.to(DEV), G, 1e-5)
    torch.cuda.synchronize()
    assert np.array_equal(p.cpu().numpy(), p_ref) and np.array_equal(sw.cpu().numpy(), s_ref)


def _grouped_bound(q, s_x, packed, s_w, G, K):
    """2^-44 (s_x / 127) sum_g |acc_g s_g| per output: the float64 sum over groups is
    taken in another order than the oracle's."""
    t = oracle.unpack(packed, K).astype(np.float64)
    sg = np.repeat(s_w.astype(np.float64), G, axis=1)
    mag = np.abs(q.astype(np.float64)) @ (np.abs(t) * sg).T
    return 2.0 ** -44 * mag * (s_x.astype(np.float64)[:, None] / 127.0)


def _gemm_group_bound(q, s_x, packed, s_w, G, K):
    """The pipelined GEMM scales each group's exact integer sum acc_g into an fp32
    accumulator: one rounding of acc_g s_g and one of each running sum, so |error| <=
    (K / G + 1) 2^-24 (s_x / 127) sum_g |acc_g s_g| before the final rounding."""
    t = oracle.unpack(packed, K).astype(np.float64)
    qf = q.astype(np.float64)
    mag = np.zeros((q.shape[0], t.shape[0]))
    for g in range(K // G):
        sl = slice(g * G, (g + 1) * G)
        mag += np.abs(qf[:, sl] @ t[:, sl].T) * s_w[:, g].astype(np.float64)[None, :]
    return (K // G + 1) * 2.0 ** -24 * mag * (s_x.astype(np.float64)[:, None] / 127.0)


@pytest.mark.parametrize("kernel,M,N,K,G", [
    (2, 257, 225, 640, 128), (21, 300, 500, 2560, 128), (22, 200, 333, 2560, 64), (0, 40, 129, 2560, 128),
    (2, 130, 96, 1024, 256), (22, 520, 1000, 1024, 512), (2, 17, 300, 6912, 128), (0, 300, 700, 2560, 640),
])
@pytest.mark.parametrize("opts", ["plain", "bias_bf16"])
def test_gemm_weight_scale_groups(kernel, M, N, K, G, opts):
    """Group-wise scales on the pipelined GEMM (no int32 output): several tiles per
    workgroup, ragged M and N, G = 64 (a group per half step) up to several steps."""
    key = synth.stream_key(337, kernel, M, N, K, G)
    x, q, s = quantized_inputs(key, M, K, row_scale=(0.1, 10.0))
    w = synth.latent_weights(synth.stream_key(key, 1), N, K, 0.02).numpy()
    w[: N // 2, :G] *= 6.0
    packed, s_w = oracle.pack_grouped(w, G, 1e-5)
    bias = (np.linspace(-2, 2, N).astype(np.float32) if opts == "bias_bf16" else None)
    _, y_ref = oracle.linear_grouped(q, s, packed, s_w, G, bias=bias)
    out_dtype = torch.bfloat16 if opts == "bias_bf16" else torch.float32
    y = torch.full((M, N), float("nan"), dtype=out_dtype, device=DEV)
    tw.bitnet_linear_ex(torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV),
                        torch.from_numpy(packed).to(DEV), torch.from_numpy(s_w).to(DEV),
                        None if bias is None else torch.from_numpy(bias).to(DEV), y, None, kernel, w_group=G)
    torch.cuda.synchronize()
    slack = _gemm_group_bound(q, s, packed, s_w, G, K)
    if out_dtype == torch.float32:
        d = np.abs(y.cpu().numpy().astype(np.float64) - y_ref.astype(np.float64))
        bad = d > REL * np.abs(y_ref.astype(np.float64)) + slack
    else:
        got = (y.cpu().view(torch.int16).numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
        want = (oracle.to_bf16(y_ref).astype(np.uint32) << 16).view(np.float32)
        d = np.abs(got.astype(np.float64) - want.astype(np.float64))
        bad = d > 2.0 ** -7 * np.abs(want.astype(np.float64)) + slack
    assert not bad.any(), f"{bad.sum()} outputs outside the bound; first at {np.argwhere(bad)[0]}"


@pytest.mark.parametrize("kernel,M,N,K,G", [
    (1, 1, 300, 2560, 2560), (4, 8, 300, 2560, 2560), (2, 40, 257, 640, 640), (3, 3, 33, 132, 132),
    (16, 257, 225, 640, 640), (17, 257, 225, 640, 640), (18, 257, 225, 640, 640), (19, 257, 225, 640, 640),
    (20, 257, 225, 640, 640), (0, 1, 640, 2560, 2560), (0, 20, 300, 2560, 2560),      # per output channel
    (1, 1, 300, 2560, 128), (1, 3, 70, 6912, 128), (1, 9, 33, 640, 64), (0, 1, 640, 2560, 128),
    (0, 20, 129, 2560, 256), (3, 4, 33, 132, 44), (0, 2, 50, 2560 + 4, 4),             # group-wise
    (1, 1, 200, 53312, 64), (1, 2, 100, 53248, 128),                                   # K in segments
    (1, 1, 16400, 640, 128), (0, 1, 16400, 640, 640),                                  # tall, one token
])
@pytest.mark.parametrize("opts", ["plain", "bias_bf16"])
def test_linear_weight_scale_groups(kernel, M, N, K, G, opts):
    key = synth.stream_key(331, kernel, M, N, K, G)
    x, q, s = quantized_inputs(key, M, K, row_scale=(0.1, 10.0))
    w = synth.latent_weights(synth.stream_key(key, 1), N, K, 0.02).numpy()
    w[: N // 2, : max(G, 4)] *= 6.0
    packed, s_w = oracle.pack_grouped(w, G, 1e-5)
    bias = (np.linspace(-2, 2, N).astype(np.float32) if opts == "bias_bf16" else None)
    acc_ref, y_ref = oracle.linear_grouped(q, s, packed, s_w, G, bias=bias)
    out_dtype = torch.bfloat16 if opts == "bias_bf16" else torch.float32
    y = torch.empty((M, N), dtype=out_dtype, device=DEV)
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    tw.bitnet_linear_ex(torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV),
                        torch.from_numpy(packed).to(DEV), torch.from_numpy(s_w).to(DEV),
                        None if bias is None else torch.from_numpy(bias).to(DEV), y, acc, kernel, w_group=G)
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    if G == K:
        # one scale per output channel: the per-tensor rescale with the row's scale
        if out_dtype == torch.float32:
            assert_y(y.cpu().numpy(), y_ref)
        else:
            assert_bf16(y.cpu().view(torch.int16).numpy().view(np.uint16), y_ref)
        return
    slack = _grouped_bound(q, s, packed, s_w, G, K)
    if bias is not None:
        slack = slack + 2.0 ** -45 * np.abs(bias.astype(np.float64))[None, :]
    if out_dtype == torch.float32:
        d = np.abs(y.cpu().numpy().astype(np.float64) - y_ref.astype(np.float64))
        bad = d > REL * np.abs(y_ref.astype(np.float64)) + slack
    else:
        got = (y.cpu().view(torch.int16).numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
        want = (oracle.to_bf16(y_ref).astype(np.uint32) << 16).view(np.float32)
        d = np.abs(got.astype(np.float64) - want.astype(np.float64))
        bad = d > 2.0 ** -7 * np.abs(want.astype(np.float64)) + slack
    assert not bad.any(), f"{bad.sum()} outputs outside the bound"


@pytest.mark.parametrize("group_acc", [True, False])
@pytest.mark.parametrize("mixed_m", [False, True, "wide"])
def test_grouped_plan_weight_scales(mixed_m, group_acc):
    """One grouped linear launch over problems with one scale per tensor, per output
    channel and per group of 128 / 64 weights (and, mixed_m, M up to 5).  group_acc
    False: the group-wise problems ask for y only, which lets the several-token kernel
    drop their integer sums; the other problems still return acc (their float64 sum is
    the integer itself)."""
    # a plain K = 51200 row (one segment of 20-dword chunks) next to group-wise rows
    shapes = [(300, 2560, 0), (129, 2560, 2560), (200, 6912, 128), (70, 640, 64), (640, 2560, 128), (64, 51200, 0)]
    probs, refs = [], []
    for i, (N, K, G) in enumerate(shapes):
        M = ([8, 16, 3, 9, 1, 12][i] if mixed_m == "wide" else (1 + i % 5)) if mixed_m else 1
        key = synth.stream_key(332, i, M)
        x, q, s = quantized_inputs(key, M, K)
        w = synth.latent_weights(synth.stream_key(key, 1), N, K, 0.02).numpy()
        w[:, : max(G, 64)] *= 5.0
        if G:
            packed, s_w = oracle.pack_grouped(w, G, 1e-5)
            acc_ref, y_ref = oracle.linear_grouped(q, s, packed, s_w, G)
            slack = _grouped_bound(q, s, packed, s_w, G, K) if G < K else None
        else:
            packed, s_w = oracle.pack(w, 1e-5)
            acc_ref, y_ref = oracle.linear(q, s, packed, s_w)
            s_w = np.array([s_w], np.float32)
            slack = None
        refs.append((acc_ref, y_ref, slack))
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        acc = torch.empty((M, N), dtype=torch.int32, device=DEV) if group_acc or not 0 < G < K else None
        probs.append((torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV), torch.from_numpy(packed).to(DEV),
                      torch.from_numpy(s_w).to(DEV), y, acc, G))
    plan = tw.bitnet_grouped_plan_linear(probs)
    for _ in range(2):
        plan.launch()
        torch.cuda.synchronize()
        for (acc_ref, y_ref, slack), pr in zip(refs, probs):
            if pr[5] is not None:
                assert np.array_equal(pr[5].cpu().numpy(), acc_ref)
            if slack is None:
                assert_y(pr[4].cpu().numpy(), y_ref)
            else:
                assert_y_within(pr[4].cpu().numpy(), y_ref, REL, slack)


# ----------------------------------------------------------------- bias and bf16 y in plans

def _bias(key, N):
    return (synth.normal(synth.stream_key(key, 21), N).float().numpy() * 0.3).astype(np.float32)


@pytest.mark.parametrize("variant", ["gemv", "groups", "mfma"])
def test_grouped_plan_bias_bf16(variant):
    """Grouped linear plans whose problems carry a bias and / or a bf16 y (each
    combination), on the plan's three kernels: the decode GEMV (M = 1), the GEMV with
    group-wise scales, the MFMA decode kernel (some M > 1).  y is the oracle's
    fp32(acc c_m + bias), bf16 rounded from it."""
    shapes = [(300, 2560, 0), (129, 6912, 0), (64, 64, 0), (700, 640, 0)]
    if variant == "groups":
        shapes += [(200, 2560, 128), (70, 640, 64)]
    opts = [(False, False), (True, False), (False, True), (True, True)]
    probs, refs = [], []
    for i, (N, K, G) in enumerate(shapes):
        M = 1 + (i % 3) if variant == "mfma" else (1 + i % 2 if variant == "groups" else 1)
        with_bias, bf16 = opts[i % 4]
        key = synth.stream_key(335, i, M)
        x, q, s = quantized_inputs(key, M, K)
        b = _bias(key, N) if with_bias else None
        if G:
            w = synth.latent_weights(synth.stream_key(key, 1), N, K, 0.02).numpy()
            packed, s_w = oracle.pack_grouped(w, G, 1e-5)
            acc_ref, y_ref = oracle.linear_grouped(q, s, packed, s_w, G, bias=b)
            slack = _grouped_bound(q, s, packed, s_w, G, K)
        else:
            packed = synth.random_bytes(synth.stream_key(key, 1), N * K // 4).numpy().reshape(N, K // 4)
            s_w = np.array([0.0043 * (i + 1)], np.float32)
            acc_ref, y_ref = oracle.linear(q, s, packed, s_w[0], bias=b)
            slack = None
        refs.append((acc_ref, y_ref, slack, bf16))
        y = torch.full((M, N), float("nan"), dtype=torch.bfloat16 if bf16 else torch.float32, device=DEV)
        acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
        probs.append((torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV), torch.from_numpy(packed).to(DEV),
                      torch.from_numpy(s_w).to(DEV), y, acc, G, None if b is None else torch.from_numpy(b).to(DEV)))
    plan = tw.bitnet_grouped_plan_linear(probs)
    for _ in range(2):
        for pr in probs:
            pr[4].fill_(float("nan"))
        plan.launch()
        torch.cuda.synchronize()
        for (acc_ref, y_ref, slack, bf16), pr in zip(refs, probs):
            assert np.array_equal(pr[5].cpu().numpy(), acc_ref)
            y = pr[4].cpu()
            if slack is not None:
                got = y.float().numpy()
                extra = 2.0 ** -8 * np.abs(y_ref.astype(np.float64)) if bf16 else 0.0
                assert_y_within(got, y_ref, REL, slack + extra)
            elif bf16:
                assert_bf16(y.view(torch.int16).numpy(), y_ref)
            else:
                assert_y(y.numpy(), y_ref)


def test_fused_plan_bias_bf16():
    """A fused plan whose rows carry a bias and / or a bf16 y: plain bf16 rows, fp32
    rows and gate / up pairs (bf16 only: a pair takes no bias)."""
    cases = [("plain", 300, 2560, True, False), ("plain", 129, 6912, False, True), ("plain", 64, 64, True, True),
             ("f32", 2560, 6912, True, True), ("f32", 97, 640, True, False), ("pair", 300, 2560, False, True),
             ("plain", 700, 2560, False, False)]
    probs, exps = [], []
    for i, (kind, N, K, with_bias, bf16) in enumerate(cases):
        key = synth.stream_key(344, i)
        xin, pw, sw, gain, exp = _fused_case(kind, N, K, key)
        b = _bias(key, N) if with_bias else None
        if b is not None:
            _, exp["y"] = oracle.linear(exp["q"], exp["s"], pw.cpu().numpy(), sw.item(), bias=b)
        y = torch.full((1, N), float("nan"), dtype=torch.bfloat16 if bf16 else torch.float32, device=DEV)
        acc = None if kind == "pair" else torch.empty((1, N), dtype=torch.int32, device=DEV)
        probs.append((xin, pw, sw, y, acc, None, None, None, 0.0, None if b is None else torch.from_numpy(b).to(DEV)))
        exps.append((kind, exp, bf16))
    plan = tw.bitnet_grouped_plan_fused(probs)
    for _ in range(2):
        for pr in probs:
            pr[3].fill_(float("nan"))
        plan.launch()
        torch.cuda.synchronize()
        for (kind, exp, bf16), pr in zip(exps, probs):
            y = pr[3].cpu()
            if kind != "pair":
                assert np.array_equal(pr[4].cpu().numpy(), exp["acc"]), kind
            if bf16:
                assert_bf16(y.view(torch.int16).numpy(), exp["y"])
            else:
                assert_y(y.numpy(), exp["y"])


# ----------------------------------------------------------------- RMSNorm + quantization

def _gain(key, K):
    g = (1.0 + 0.25 * synth.normal(synth.stream_key(key, 11), K).float().numpy()).astype(np.float32)
    g[::5] = -g[::5]
    return g


def assert_scale(s_gpu, s_ref):
    """The scale of a normalized row: within one fp32 unit (the sum of squares is
    taken in float64 in another order than the oracle's)."""
    s_gpu = s_gpu.astype(np.float64)
    s_ref = s_ref.astype(np.float64)
    assert np.all(np.abs(s_gpu - s_ref) <= 2.0 ** -23 * np.abs(s_ref)), "scale more than one unit away"


@pytest.mark.parametrize("M,K,kw,eps", [(1, 2560, {}, 1e-6), (5, 6912, {"outlier_frac": 0.001}, 1e-5),
                                        (3, 64, {}, 0.0), (17, 640, {"row_scale": (1e-3, 1e3)}, 1e-6),
                                        (2, 52224, {"outlier_frac": 0.01}, 1e-6)])
def test_rmsnorm_quant_parity(M, K, kw, eps):
    key = synth.stream_key(320, M, K)
    x = synth.activations(key, M, K, **kw)
    if M > 2:
        x[1].zero_()
    g = _gain(key, K)
    q_ref, s_ref = oracle.rmsnorm_quant(bits_np(x), g, eps)
    q, s = tw.rmsnorm_quant(x.to(DEV), torch.from_numpy(g).to(DEV), eps)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert_scale(s.cpu().numpy(), s_ref)


@pytest.mark.parametrize("with_outputs", [True, False])
def test_fused_rmsnorm_linear_grouped(with_outputs):
    """One fused launch mixing problems with and without an RMSNorm: codes and acc
    exact, the scale within one fp32 unit, y within 2^-22 (the scale's unit plus the
    rescale's rounding) of the oracle's rmsnorm_quant + linear."""
    shapes = [(300, 2560, True), (640, 2560, True), (97, 6912, False), (129, 12288, True), (64, 64, True),
              (200, 2560, False), (33, 2560, "zero")]
    probs, refs = [], []
    for i, (N, K, norm) in enumerate(shapes):
        key = synth.stream_key(321, i)
        x = torch.zeros((1, K), dtype=torch.bfloat16) if norm == "zero" else synth.activations(key, 1, K, outlier_frac=0.002)
        packed = synth.random_bytes(synth.stream_key(key, 1), N * K // 4).numpy().reshape(N, K // 4)
        s_w = np.float32(0.0071 * (i + 1))
        if norm:
            g = _gain(key, K)
            q_ref, sx_ref = oracle.rmsnorm_quant(bits_np(x), g, 1e-6)
        else:
            g = None
            q_ref, sx_ref = oracle.quant_act(bits_np(x))
        acc_ref, y_ref = oracle.linear(q_ref, sx_ref, packed, s_w)
        refs.append((q_ref, sx_ref, acc_ref, y_ref, bool(norm)))
        y = torch.full((1, N), float("nan"), dtype=torch.float32, device=DEV)
        acc = torch.empty((1, N), dtype=torch.int32, device=DEV)
        q = torch.full((1, K), 99, dtype=torch.int8, device=DEV) if with_outputs else None
        sx = torch.full((1,), -1.0, dtype=torch.float32, device=DEV) if with_outputs else None
        probs.append((x.to(DEV), torch.from_numpy(packed).to(DEV), torch.tensor([s_w], device=DEV), y, acc, q, sx,
                      None if g is None else torch.from_numpy(g).to(DEV), 1e-6))
    plan = tw.bitnet_grouped_plan_fused(probs)
    for _ in range(2):
        for pr in probs:
            pr[3].fill_(float("nan"))
            pr[4].fill_(-1)
        plan.launch()
        torch.cuda.synchronize()
        for (q_ref, sx_ref, acc_ref, y_ref, norm), pr in zip(refs, probs):
            assert np.array_equal(pr[4].cpu().numpy(), acc_ref)
            if norm:
                assert_y_within(pr[3].cpu().numpy(), y_ref, 2.0 ** -22)
            else:
                assert_y(pr[3].cpu().numpy(), y_ref)
            if with_outputs:
                assert np.array_equal(pr[5].cpu().numpy(), q_ref)
                assert_scale(pr[6].cpu().numpy(), sx_ref)


# ----------------------------------------------------------------- SwiGLU + quantization

def _gate_up(key, M, K, outliers=False):
    """Gate and up outputs: normal rows (gate wider, so that silu's bend and both
    tails are hit), a few large values when asked."""
    g = (3.0 * synth.normal(synth.stream_key(key, 1), M * K).float().numpy()).astype(np.float32).reshape(M, K)
    u = synth.normal(synth.stream_key(key, 2), M * K).float().numpy().astype(np.float32).reshape(M, K)
    if outliers:
        g[:, ::997] *= 8.0
        u[:, 5::1009] *= 20.0
    return g, u


@pytest.mark.parametrize("M,K,outliers", [(1, 6912, False), (4, 6912, True), (3, 64, False), (2, 8, False),
                                          (5, 27648, True), (1, 52224, False), (33, 2560, False)])
def test_swiglu_quant_parity(M, K, outliers):
    key = synth.stream_key(340, M, K)
    g, u = _gate_up(key, M, K, outliers)
    if M > 2:
        u[1] = 0.0          # a row of zeros after SwiGLU
    _, q_ref, s_ref = oracle.swiglu_quant(g, u)
    q, s = tw.swiglu_quant(torch.from_numpy(g).to(DEV), torch.from_numpy(u).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


def _near_tie_row(K, key):
    """fp32 row whose values sit within an fp32 rounding of code boundaries for the
    row scale 1 (x = fl((2j + 1) / 254)), mixed with normal values below it."""
    x = (0.3 * synth.normal(key, K).float().numpy()).astype(np.float32)
    x = np.clip(x, -0.99, 0.99)
    j = np.arange(K) % 127
    x[::3] = (((2 * j + 1) / 254.0) * np.where(j % 2, 1.0, -1.0)).astype(np.float32)[::3]
    x[K // 2] = 1.0
    return x.reshape(1, K)


def _fused_case(kind, N, K, key):
    """Inputs and the oracle's expected outputs of one fused problem of a kind:
    'plain' / 'norm' (bf16 row), 'f32' / 'f32tie' / 'f32zero' (fp32 row), 'pair' /
    'pairnorm' (gate / up pair)."""
    pk = lambda k: synth.random_bytes(synth.stream_key(key, k), N * K // 4).numpy().reshape(N, K // 4)
    s_w = np.float32(0.0037 + 0.001 * (key % 7))
    gain = None
    if kind.startswith("f32"):
        if kind == "f32tie":
            x = _near_tie_row(K, synth.stream_key(key, 5))
        elif kind == "f32zero":
            x = np.zeros((1, K), np.float32)
        else:
            x = (synth.normal(synth.stream_key(key, 5), K).float().numpy() * 0.7).astype(np.float32).reshape(1, K)
            x[0, ::501] *= 30.0
        q_ref, sx_ref = oracle.quant_act_f32(x)
        xin = torch.from_numpy(x).to(DEV)
    else:
        x = synth.activations(synth.stream_key(key, 6), 1, K, outlier_frac=0.002)
        if kind in ("norm", "pairnorm"):
            gn = _gain(key, K)
            q_ref, sx_ref = oracle.rmsnorm_quant(bits_np(x), gn, 1e-6)
            gain = torch.from_numpy(gn).to(DEV)
        else:
            q_ref, sx_ref = oracle.quant_act(bits_np(x))
        xin = x.to(DEV)
    packed = pk(1)
    if kind.startswith("pair"):
        packed_up = pk(2)
        s_up = np.float32(s_w * 1.7)
        _, y_g = oracle.linear(q_ref, sx_ref, packed, s_w)
        _, y_u = oracle.linear(q_ref, sx_ref, packed_up, s_up)
        a_ref = oracle.swiglu_quant(y_g, y_u)[0]
        exp = dict(q=q_ref, s=sx_ref, y=a_ref, acc=None, gu=(y_g, y_u))
        pw = (torch.from_numpy(packed).to(DEV), torch.from_numpy(packed_up).to(DEV))
        sw = (torch.tensor([s_w], device=DEV), torch.tensor([s_up], device=DEV))
    else:
        acc_ref, y_ref = oracle.linear(q_ref, sx_ref, packed, s_w)
        exp = dict(q=q_ref, s=sx_ref, y=y_ref, acc=acc_ref)
        pw, sw = torch.from_numpy(packed).to(DEV), torch.tensor([s_w], device=DEV)
    return xin, pw, sw, gain, exp


def swiglu_pair_bound(y_g, y_u, rel):
    """How far a = silu(g) u can move when g and u each move by rel of themselves:
    |d a| <= |silu'(g)| |g| rel |u| + |silu(g)| |u| rel, plus one fp32 rounding of a."""
    g = y_g.astype(np.float64)
    u = y_u.astype(np.float64)
    sg = 1.0 / (1.0 + np.exp(-g))
    dsilu = sg * (1.0 + g * (1.0 - sg))
    a = g * sg * u
    return 2 * rel * (np.abs(dsilu * g * u) + np.abs(a)) + 2.0 ** -23 * np.abs(a)


def _check_fused(kind, exp, y, acc, q, sx):
    if kind == "pair":
        # y_gate and y_up match the oracle's bit for bit (the same float64 factor and
        # product, one rounding each), so does a = fp32(silu(y_gate) y_up)
        assert np.array_equal(y, exp["y"]), kind
    elif kind == "pairnorm":
        # the RMSNorm scale s_x may sit one fp32 unit from the oracle's, which moves
        # y_gate and y_up by up to 2^-22 of themselves
        bound = swiglu_pair_bound(exp["gu"][0], exp["gu"][1], 2.0 ** -22)
        assert np.all(np.abs(y.astype(np.float64) - exp["y"].astype(np.float64)) <= bound), kind
    else:
        assert np.array_equal(acc, exp["acc"]), kind
        if kind == "norm":
            assert_y_within(y, exp["y"], 2.0 ** -22)
        else:
            assert_y(y, exp["y"])
    if q is not None:
        assert np.array_equal(q, exp["q"]), kind
        if kind in ("norm", "pairnorm"):
            assert_scale(sx, exp["s"])
        else:
            assert np.array_equal(sx, exp["s"]), kind


FUSED_SWIGLU_SHAPES = [("pairnorm", 6912, 2560), ("pair", 300, 2560), ("pair", 65, 64), ("pairnorm", 1, 12288),
                       ("f32", 2560, 6912), ("f32tie", 97, 12288), ("f32", 129, 52224), ("f32", 64, 64),
                       ("f32zero", 33, 6912), ("norm", 300, 2560), ("plain", 200, 2560)]


@pytest.mark.parametrize("with_outputs", [True, False])
def test_fused_swiglu_ends(with_outputs):
    """One fused launch with gate / up pairs (SwiGLU epilogue) and fp32 input rows
    (the down projections) next to plain and RMSNorm rows; then the same problems
    without the RMSNorm ones (the kernel without that path)."""
    probs, cases = [], []
    for i, (kind, N, K) in enumerate(FUSED_SWIGLU_SHAPES):
        xin, pw, sw, gain, exp = _fused_case(kind, N, K, synth.stream_key(342, i))
        y = torch.full((1, N), float("nan"), dtype=torch.float32, device=DEV)
        acc = None if kind.startswith("pair") else torch.empty((1, N), dtype=torch.int32, device=DEV)
        q = torch.full((1, K), 99, dtype=torch.int8, device=DEV) if with_outputs else None
        sx = torch.full((1,), -1.0, dtype=torch.float32, device=DEV) if with_outputs else None
        probs.append((xin, pw, sw, y, acc, q, sx, gain, 1e-6))
        cases.append((kind, exp))
    for sel in (range(len(probs)), [i for i, c in enumerate(cases) if "norm" not in c[0]]):
        sub = [probs[i] for i in sel]
        plan = tw.bitnet_grouped_plan_fused(sub)
        for rep in range(2):
            for pr in sub:
                pr[3].fill_(float("nan"))
                if pr[4] is not None:
                    pr[4].fill_(-1)
            plan.launch()
            torch.cuda.synchronize()
            for i in sel:
                pr = probs[i]
                kind, exp = cases[i]
                _check_fused(kind, exp, pr[3].cpu().numpy(), None if pr[4] is None else pr[4].cpu().numpy(),
                             None if pr[5] is None else pr[5].cpu().numpy(),
                             None if pr[6] is None else pr[6].cpu().numpy())


def test_fused_pair_matches_swiglu_then_linear():
    """The pair's output fed back as an fp32 row gives the codes that
    bitnet_swiglu_quant_act gives from the two projections' outputs."""
    N, K, Nd = 6912, 2560, 2560
    key = synth.stream_key(343)
    x = synth.activations(key, 1, K).to(DEV)
    pg = torch.from_numpy(synth.random_bytes(synth.stream_key(key, 1), N * K // 4).numpy().reshape(N, K // 4)).to(DEV)
    pu = torch.from_numpy(synth.random_bytes(synth.stream_key(key, 2), N * K // 4).numpy().reshape(N, K // 4)).to(DEV)
    sg, su = torch.tensor([0.011], device=DEV), torch.tensor([0.017], device=DEV)
    a = torch.empty((1, N), dtype=torch.float32, device=DEV)
    tw.bitnet_grouped_plan_fused([(x, (pg, pu), (sg, su), a, None, None, None)]).launch()
    q, s = tw.quant_act(x)
    yg = tw.linear(q, s, pg, sg)
    yu = tw.linear(q, s, pu, su)
    q2, s2 = tw.swiglu_quant(yg, yu)
    pd = torch.from_numpy(synth.random_bytes(synth.stream_key(key, 3), Nd * N // 4).numpy().reshape(Nd, N // 4)).to(DEV)
    yd = torch.empty((1, Nd), dtype=torch.float32, device=DEV)
    qa = torch.empty((1, N), dtype=torch.int8, device=DEV)
    sa = torch.empty((1,), dtype=torch.float32, device=DEV)
    tw.bitnet_grouped_plan_fused([(a, pd, sg, yd, None, qa, sa)]).launch()
    torch.cuda.synchronize()
    assert torch.equal(qa, q2) and torch.equal(sa, s2)


# ----------------------------------------------------------------- binary weights, sign / mask bitplanes

@pytest.mark.parametrize("N,K", [(300, 2560), (33, 6912), (5, 32), (70, 640)])
def test_pack_binary_parity(N, K):
    w = synth.latent_weights(synth.stream_key(350, N, K), N, K, 0.02)
    w[0, :7] = 0.0
    w[1, :3] = -0.0
    b_ref, s_ref = oracle.pack_binary(w.numpy())
    bits, s_w = tw.pack_weights_binary(w.to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(bits.cpu().numpy(), b_ref) and s_w.item() == s_ref


@pytest.mark.parametrize("N,K", [(300, 2560), (7, 32), (129, 6912)])
def test_pack_bitplanes_parity(N, K):
    packed = synth.random_bytes(synth.stream_key(351, N, K), N * K // 4).numpy().reshape(N, K // 4)  # codes 0-3
    ref = oracle.pack_bitplanes(packed, K)
    planes = tw.pack_bitplanes(torch.from_numpy(packed).to(DEV), K)
    torch.cuda.synchronize()
    assert np.array_equal(planes.cpu().numpy(), ref)


def _bits_case(fmt, N, K, key):
    if fmt == tw.FMT_BINARY:
        wb = synth.random_bytes(synth.stream_key(key, 1), N * K // 8).numpy().reshape(N, K // 8)
        return wb, lambda q, s, sw: oracle.linear_binary(q, s, wb, sw)
    w = synth.latent_weights(synth.stream_key(key, 1), N, K, 0.02).numpy()
    packed, _ = oracle.pack(w)
    wb = oracle.pack_bitplanes(packed, K)
    return wb, lambda q, s, sw: oracle.linear_bitplanes(q, s, wb, sw)


BITS_SHAPES = [(1, 300, 2560), (1, 2560, 6912), (1, 65, 128), (1, 1, 256), (1, 700, 8192), (1, 129, 28672),
               (1, 16400, 640), (1, 16384, 8192), (3, 70, 640), (8, 33, 2560),
               # several tokens per pass (4 / 2 / 1 by K and format), ragged token tiles
               (2, 300, 2560), (5, 129, 6912), (16, 1000, 8192), (4, 64, 28672), (9, 70, 640), (7, 65, 128)]


@pytest.mark.parametrize("fmt", [1, 2])
@pytest.mark.parametrize("M,N,K", BITS_SHAPES)
def test_linear_bits_parity(fmt, M, N, K):
    key = synth.stream_key(352, fmt, M, N, K)
    x, q, s = quantized_inputs(key, M, K, outlier_frac=0.002)
    wb, ref = _bits_case(fmt, N, K, key)
    s_w = np.float32(0.0123)
    acc_ref, y_ref = ref(q, s, s_w)
    qd, sd = torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV)
    wd, swd = torch.from_numpy(wb).to(DEV), torch.tensor([s_w], device=DEV)
    kernels = ((0, 1, 2, 3) if M == 1 else (0, 1, 3)) + ((4,) if K % 64 == 0 else ())
    for kern in kernels:
        y, acc = tw.linear_bits(qd, sd, wd, fmt, swd, want_acc=True, kernel=kern)
        torch.cuda.synchronize()
        assert np.array_equal(acc.cpu().numpy(), acc_ref), kern
        assert_y(y.cpu().numpy(), y_ref)


@pytest.mark.parametrize("fmt", [1, 2])
@pytest.mark.parametrize("M,N,K", [(2, 1, 64), (16, 5000, 2560), (17, 300, 6912), (40, 129, 1024), (8, 6000, 8192),
                                   (3, 7, 28672), (33, 4096, 128), (8, 65, 57344), (4, 131112, 128),
                                   (3, 262200, 64), (8, 40000, 8192), (20, 131080, 256), (8, 131072, 6912)])
def test_linear_bits_mfma(fmt, M, N, K):
    """The matrix-core kernel for binary weights and bitplanes (kernel 4): one to three
    16-token tiles, ragged rows, K split over 1 to 8 wavefronts, one, two or four
    16-row groups per wavefront, from 131072 rows the form with q staged once per
    workgroup (K in segments, a ragged second token tile), K from one chunk to 57344,
    random weight bits (binary) or
    planes of random 2-bit codes (code 3 as +1), and a token row of +-127 so that every
    byte of the products counts; acc bit-exact and y against the oracle's product over
    the same weights."""
    key = synth.stream_key(354, fmt, M, N, K)
    x, q, s = quantized_inputs(key, M, K, outlier_frac=0.002)
    q[0, ::2] = 127
    q[0, 1::2] = -127
    s[0] = np.float32(1.5)
    s_w = np.float32(0.0109)
    if fmt == tw.FMT_BINARY:
        wb = synth.random_bytes(synth.stream_key(key, 1), N * K // 8).numpy().reshape(N, K // 8)
        acc_ref, y_ref = oracle.linear_binary(q, s, wb, s_w)
    else:
        packed = synth.random_bytes(synth.stream_key(key, 1), N * K // 4).numpy().reshape(N, K // 4)
        wb = oracle.pack_bitplanes(packed, K)
        acc_ref, y_ref = oracle.linear_bitplanes(q, s, wb, s_w)
    y, acc = tw.linear_bits(torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV), torch.from_numpy(wb).to(DEV),
                            fmt, torch.tensor([s_w], device=DEV), want_acc=True, kernel=4)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert_y(y.cpu().numpy(), y_ref)


@pytest.mark.parametrize("N", [97, 16400])
@pytest.mark.parametrize("fmt,K", [(1, 57344), (2, 51584)])
def test_linear_bits_longest_k(fmt, K, N):
    """The longest K whose staged planes fit LDS, with extreme codes (+-127, -127 on
    every value of one row) so that every plane and the sign plane count; N below
    and above the row count where the kernel takes 4 rows per octet."""
    key = synth.stream_key(353, fmt, K)
    q = np.full((1, K), -127, np.int8)
    q[0, ::3] = 127
    q[0, 5::7] = 0
    s = np.array([0.75], np.float32)
    wb, ref = _bits_case(fmt, N, K, key)
    acc_ref, y_ref = ref(q, s, np.float32(0.01))
    y, acc = tw.linear_bits(torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV), torch.from_numpy(wb).to(DEV),
                            fmt, torch.tensor([0.01], device=DEV), want_acc=True, kernel=2)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert_y(y.cpu().numpy(), y_ref)


@pytest.mark.parametrize("with_outputs", [True, False])
def test_fused_bitplanes_grouped(with_outputs):
    """The fused decode plan over bitplane weights against the oracle's quant_act +
    linear of the same 2-bit codes: ragged N, K from one slot to the longest bitplane
    K, an all-zero row, outliers."""
    shapes = [(2560, 6912, {}), (300, 2560, {"outlier_frac": 0.01}), (129, 51584, {}), (64, 64, {}),
              (700, 8192, {"row_scale": (1e-3, 1e-3)}), (33, 2560, "zero"), (1, 128, {})]
    probs, refs = [], []
    for i, (N, K, kw) in enumerate(shapes):
        key = synth.stream_key(355, i)
        x = torch.zeros((1, K), dtype=torch.bfloat16) if kw == "zero" else synth.activations(key, 1, K, **kw)
        w = synth.latent_weights(synth.stream_key(key, 1), N, K, 0.02).numpy()
        packed, s_w = oracle.pack(w)
        q_ref, sx_ref = oracle.quant_act(bits_np(x))
        acc_ref, y_ref = oracle.linear(q_ref, sx_ref, packed, s_w)
        refs.append((q_ref, sx_ref, acc_ref, y_ref))
        planes = torch.from_numpy(oracle.pack_bitplanes(packed, K)).to(DEV)
        y = torch.full((1, N), float("nan"), dtype=torch.float32, device=DEV)
        acc = torch.empty((1, N), dtype=torch.int32, device=DEV)
        q = torch.full((1, K), 99, dtype=torch.int8, device=DEV) if with_outputs else None
        sx = torch.full((1,), -1.0, dtype=torch.float32, device=DEV) if with_outputs else None
        probs.append((x.to(DEV), planes, torch.tensor([s_w], device=DEV), y, acc, q, sx))
    plan = tw.bitnet_grouped_plan_fused(probs)
    for _ in range(2):
        for pr in probs:
            pr[3].fill_(float("nan"))
            pr[4].fill_(-1)
        plan.launch()
        torch.cuda.synchronize()
        for (q_ref, sx_ref, acc_ref, y_ref), pr in zip(refs, probs):
            assert np.array_equal(pr[4].cpu().numpy(), acc_ref)
            assert_y(pr[3].cpu().numpy(), y_ref)
            if with_outputs:
                assert np.array_equal(pr[5].cpu().numpy(), q_ref)
                assert np.array_equal(pr[6].cpu().numpy(), sx_ref)


def test_bitplanes_equal_two_bit_codes_on_gpu():
    """The same ternary weights through the 2-bit GEMV and the bitplane GEMV."""
    N, K = 2560, 6912
    key = synth.stream_key(354)
    x, q, s = quantized_inputs(key, 1, K)
    w = synth.latent_weights(synth.stream_key(key, 1), N, K, 0.02)
    packed, s_w = tw.pack_weights(w.to(DEV))
    planes = tw.pack_bitplanes(packed, K)
    qd, sd = torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV)
    y2, a2 = tw.linear(qd, sd, packed, s_w, want_acc=True)
    yb, ab = tw.linear_bits(qd, sd, planes, tw.FMT_BITPLANES, s_w, want_acc=True)
    torch.cuda.synchronize()
    assert torch.equal(a2, ab) and torch.equal(y2, yb)


@pytest.mark.parametrize("M,N,K", [(1, 200, 53312), (2, 70, 26176), (3, 200, 16704), (8, 200, 16704),
                                   (13, 130, 8192), (16, 65, 28672)])
def test_gemv_parity_k_segments(M, N, K):
    # K long enough that the staged q tile of the M tile exceeds the LDS budget, so
    # the GEMV walks K in segments (uneven last segment, ragged N).
    key = synth.stream_key(302, M, N, K)
    x, q, s = quantized_inputs(key, M, K)
    w = synth.latent_weights(synth.stream_key(key, 1), N, K, 0.02)
    packed, s_w = oracle.pack(w.numpy())
    check_linear(q, s, packed, s_w, kernels=(0, 1))


@pytest.mark.parametrize("shapes", [
    # M = 1 everywhere: the GEMV variant; one K needs two LDS segments
    [(1, 300, 2560), (1, 129, 53312), (1, 64, 64), (1, 97, 6912), (1, 700, 640)],
    # some M > 1: the MFMA variant for every problem, M = 1 included
    [(1, 300, 2560), (3, 129, 53312), (1, 64, 64), (16, 97, 6912), (2, 700, 640)],
])
def test_grouped_linear_mixed_k(shapes):
    """One grouped launch over problems with different M, N and K; every output is
    compared."""
    probs, refs = [], []
    for i, (M, N, K) in enumerate(shapes):
        key = synth.stream_key(303, i)
        x, q, s = quantized_inputs(key, M, K)
        packed = synth.random_bytes(synth.stream_key(key, 1), N * K // 4).numpy().reshape(N, K // 4)
        s_w = np.float32(0.0071 * (i + 1))
        refs.append(oracle.linear(q, s, packed, s_w))
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
        probs.append((torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV), torch.from_numpy(packed).to(DEV),
                      torch.tensor([s_w], dtype=torch.float32, device=DEV), y, acc))
    plan = tw.bitnet_grouped_plan_linear(probs)
    # several launches of one plan in stream order (the GEMV variant's work counters
    # must be back at zero after each launch), outputs cleared in between
    for _ in range(3):
        for pr in probs:
            pr[4].fill_(float("nan"))
            pr[5].fill_(-1)
        plan.launch()
        torch.cuda.synchronize()
        for (acc_ref, y_ref), pr in zip(refs, probs):
            assert np.array_equal(pr[5].cpu().numpy(), acc_ref)
            assert_y(pr[4].cpu().numpy(), y_ref)


@pytest.mark.parametrize("M,N,K", [(17, 129, 256), (32, 300, 2560), (64, 6912, 2560), (130, 257, 640),
                                   (200, 96, 6912), (2048, 384, 2560)])
def test_gemm_parity(M, N, K):
    """The MFMA GEMM, forced (the automatic choice takes the MFMA decode kernel for
    some of these shapes)."""
    key = synth.stream_key(302, M, N, K)
    x, q, s = quantized_inputs(key, M, K, row_scale=(0.1, 10.0))
    packed = synth.random_bytes(synth.stream_key(key, 1), N * K // 4).numpy().reshape(N, K // 4)
    acc_ref, y_ref = oracle.linear(q, s, packed, np.float32(0.0071))
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    tw.bitnet_linear_select(torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV),
                            torch.from_numpy(packed).to(DEV), torch.tensor([0.0071], device=DEV), y, acc, 2)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert_y(y.cpu().numpy(), y_ref)


@pytest.mark.parametrize("M,N,K", [(17, 2560, 2560), (48, 640, 6912), (96, 300, 2560), (130, 257, 640),
                                   (256, 2560, 6912), (256, 6912, 2560)])
def test_linear_auto_dispatch_beyond_16_tokens(M, N, K):
    """bitnet_linear's own choice between the MFMA decode kernel and the GEMM for
    M > 16 (an estimate of each): parity whichever it takes."""
    key = synth.stream_key(309, M, N, K)
    x, q, s = quantized_inputs(key, M, K, row_scale=(0.1, 10.0))
    packed = synth.random_bytes(synth.stream_key(key, 1), N * K // 4).numpy().reshape(N, K // 4)
    check_linear(q, s, packed, np.float32(0.0093))


@pytest.mark.parametrize("cfg,M,N,K", [(5, 1100, 6912, 128), (6, 1300, 4000, 256), (5, 520, 7000, 128),
                                       (6, 2048, 2560 + 16, 128), (5, 300, 500, 6912 - 128)])
def test_gemm_pipelined_several_tiles_per_workgroup(cfg, M, N, K):
    """The pipelined GEMM with more tiles than workgroups: each workgroup walks its
    tiles in one step sequence, loads of the next tile overlapping the current one,
    ragged last M and N tiles, K of one to three steps."""
    key = synth.stream_key(315, cfg, M, N, K)
    x, q, s = quantized_inputs(key, M, K, row_scale=(0.1, 10.0))
    packed = synth.random_bytes(synth.stream_key(key, 1), N * K // 4).numpy().reshape(N, K // 4)
    acc_ref, y_ref = oracle.linear(q, s, packed, np.float32(0.0077))
    args = (torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV), torch.from_numpy(packed).to(DEV),
            torch.tensor([0.0077], device=DEV))
    for rep in range(2):
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        acc = torch.full((M, N), -1, dtype=torch.int32, device=DEV)
        tw.bitnet_linear_select(*args, y, acc if rep == 0 else None, 16 + cfg)
        torch.cuda.synchronize()
        if rep == 0:
            assert np.array_equal(acc.cpu().numpy(), acc_ref)
        assert_y(y.cpu().numpy(), y_ref)


@pytest.mark.parametrize("cfg", range(7))
@pytest.mark.parametrize("M,N,K", [(300, 500, 640), (17, 33, 64), (257, 225, 6912 - 64), (5, 230, 256),
                                   (1, 1, 128)])
def test_gemm_tile_configs(cfg, M, N, K):
    """Every MFMA tile configuration, forced, on ragged M and N, down to a single row
    and column (the tiles whose staging repeats the last row past M or N)."""
    key = synth.stream_key(307, M, N, K)
    x, q, s = quantized_inputs(key, M, K, row_scale=(0.1, 10.0))
    packed = synth.random_bytes(synth.stream_key(key, 1), N * K // 4).numpy().reshape(N, K // 4)
    acc_ref, y_ref = oracle.linear(q, s, packed, np.float32(0.0093))
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    tw.bitnet_linear_select(torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV),
                            torch.from_numpy(packed).to(DEV), torch.tensor([0.0093], device=DEV),
                            y, acc, 16 + cfg)
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert_y(y.cpu().numpy(), y_ref)


# ----------------------------------------------------------------- epilogue options

@pytest.mark.parametrize("cfg", [2, 16, 17, 18, 19, 20, 21, 22])
@pytest.mark.parametrize("M,N,K,with_bias", [(257, 225, 640, False), (300, 500, 640, True),
                                             (130, 258, 6912 - 64, True), (2048, 384, 2560, False)])
def test_gemm_output_without_acc(cfg, M, N, K, with_bias):
    """The GEMM's output written without the int32 accumulators: fp32 bit-identical
    to the same call that also returns acc and to the oracle; bf16 equal to that fp32
    result rounded to nearest even; N not a multiple of 4, or y only 4-byte aligned,
    takes the element-wise stores."""
    key = synth.stream_key(313, cfg, M, N, K)
    x, q, s = quantized_inputs(key, M, K, row_scale=(0.1, 10.0))
    packed = synth.random_bytes(synth.stream_key(key, 1), N * K // 4).numpy().reshape(N, K // 4)
    s_w = np.float32(0.0081)
    bias = None
    if with_bias:
        bias = synth.activations(synth.stream_key(key, 2), 1, N).float().numpy()[0] * np.float32(3.0)
    acc_ref, y_ref = oracle.linear(q, s, packed, s_w, bias=bias)
    args = (torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV), torch.from_numpy(packed).to(DEV),
            torch.tensor([s_w], device=DEV), None if bias is None else torch.from_numpy(bias).to(DEV))
    y_acc = torch.empty((M, N), dtype=torch.float32, device=DEV)
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    tw.bitnet_linear_ex(*args, y_acc, acc, cfg)
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    want32 = y_acc.cpu()
    assert_y(want32.numpy(), y_ref)
    for dtype in (torch.float32, torch.bfloat16):
        for offset in (0, 4 // dtype.itemsize):     # y 4 bytes past an aligned address
            buf = torch.full((M * N + offset,), float("nan"), dtype=dtype, device=DEV)
            y = buf[offset:].view(M, N)
            tw.bitnet_linear_ex(*args, y, None, cfg)
            got = y.cpu()
            want = want32 if dtype == torch.float32 else want32.to(torch.bfloat16)
            assert torch.equal(got.view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                               want.view(torch.int16 if dtype == torch.bfloat16 else torch.int32)), (dtype, offset)


@pytest.mark.parametrize("kernel,M,N,K", [
    (1, 1, 300, 2560), (1, 3, 70, 6912), (1, 9, 33, 640),             # decode GEMV
    (4, 2, 300, 2624), (4, 16, 129, 2560), (4, 20, 70, 640),           # MFMA decode
    (2, 17, 129, 256), (2, 130, 257, 640),                             # MFMA GEMM, automatic tile
    (16, 257, 225, 640), (17, 257, 225, 640), (18, 257, 225, 640),     # each forced tile
    (19, 257, 225, 640), (20, 257, 225, 640), (21, 257, 225, 640), (22, 257, 225, 640),
    (3, 3, 9, 68), (3, 20, 33, 132),                                   # general kernel
    (0, 1, 640, 2560), (0, 8, 300, 2560), (0, 40, 300, 2560),          # automatic choice
])
@pytest.mark.parametrize("with_bias,out_dtype", [(True, torch.float32), (False, torch.bfloat16),
                                                 (True, torch.bfloat16)])
def test_linear_epilogue_options(kernel, M, N, K, with_bias, out_dtype):
    """bitnet_linear_ex: the bias added after the rescale and the bf16 output,
    on every kernel; acc is unchanged by either option."""
    key = synth.stream_key(311, kernel, M, N, K)
    x, q, s = quantized_inputs(key, M, K, row_scale=(0.1, 10.0))
    w = synth.latent_weights(synth.stream_key(key, 1), N, K, 0.02).numpy()
    packed, s_w = oracle.pack(w)
    bias = None
    if with_bias:
        bias = synth.activations(synth.stream_key(key, 2), 1, N).float().numpy()[0] * np.float32(3.0)
    acc_ref, y_ref = oracle.linear(q, s, packed, s_w, bias=bias)
    y = torch.empty((M, N), dtype=out_dtype, device=DEV)
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    tw.bitnet_linear_ex(torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV),
                        torch.from_numpy(packed).to(DEV), torch.tensor([s_w], device=DEV),
                        None if bias is None else torch.from_numpy(bias).to(DEV), y, acc, kernel)
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    if out_dtype == torch.float32:
        assert_y(y.cpu().numpy(), y_ref)
        return
    # bf16: the oracle's fp32 y rounded to nearest even
    yb = y.cpu().view(torch.int16).numpy().view(np.uint16)
    assert_bf16(yb, y_ref)
    # and the bf16 output is exactly the library's own fp32 result rounded to nearest even
    y32 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    tw.bitnet_linear_ex(torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV),
                        torch.from_numpy(packed).to(DEV), torch.tensor([s_w], device=DEV),
                        None if bias is None else torch.from_numpy(bias).to(DEV), y32, None, kernel)
    rne = y32.cpu().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(yb, rne)


def test_linear_ex_without_options_matches_linear():
    """bias = NULL and fp32 output: bit-identical to bitnet_linear."""
    M, N, K = 5, 300, 2560
    key = synth.stream_key(312)
    x, q, s = quantized_inputs(key, M, K)
    packed = synth.random_bytes(synth.stream_key(key, 1), N * K // 4).numpy().reshape(N, K // 4)
    args = (torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV), torch.from_numpy(packed).to(DEV),
            torch.tensor([0.011], device=DEV))
    y1 = tw.linear(*args)
    y2 = torch.empty_like(y1)
    tw.bitnet_linear_ex(*args, None, y2, None, 0)
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("M,N,K", [(1, 5, 4), (3, 9, 68), (20, 33, 132), (2, 70, 2560 + 4)])
def test_generic_path_parity(M, N, K):
    key = synth.stream_key(303, M, N, K)
    x, q, s = quantized_inputs(key, M, K)
    packed = synth.random_bytes(synth.stream_key(key, 1), N * K // 4).numpy().reshape(N, K // 4)
    check_linear(q, s, packed, np.float32(0.02))


def test_unaligned_q_takes_general_path():
    M, N, K = 3, 50, 640
    key = synth.stream_key(304)
    x, q, s = quantized_inputs(key, M, K)
    packed = synth.random_bytes(synth.stream_key(key, 1), N * K // 4).numpy().reshape(N, K // 4)
    acc_ref, y_ref = oracle.linear(q, s, packed, np.float32(0.5))
    big = torch.zeros(M * K + 1, dtype=torch.int8, device=DEV)
    big[1:] = torch.from_numpy(q).reshape(-1).to(DEV)
    qv = big[1:].view(M, K)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    acc = torch.empty((M, N), dtype=torch.int32, device=DEV)
    tw.bitnet_linear(qv, torch.from_numpy(s).to(DEV), torch.from_numpy(packed).to(DEV),
                     torch.tensor([0.5], device=DEV), y, acc)
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert_y(y.cpu().numpy(), y_ref)


@pytest.mark.parametrize("M", [1, 8, 40])
def test_linear_degenerate_inputs(M):
    N, K = 200, 1024
    key = synth.stream_key(305, M)
    x = synth.activations(key, M, K)
    x[M // 2] = 0                                     # an all-zero token
    q, s = oracle.quant_act(bits_np(x))
    zero_w = np.full((N, K // 4), 0x55, np.uint8)    # all-zero weights
    acc, y = check_linear(q, s, zero_w, np.float32(0.0))
    assert np.all(acc == 0) and np.all(y == 0)
    three = np.full((N, K // 4), 0xFF, np.uint8)     # code 3 everywhere -> +2
    acc3, y3 = check_linear(q, s, three, np.float32(1.0))
    assert np.array_equal(acc3[:, 0], 2 * q.astype(np.int64).sum(1))
    assert np.all(y3[M // 2] == 0)


def test_empty_problems_are_noops():
    y = torch.full((0, 5), 1.0, device=DEV)
    tw.bitnet_linear(torch.empty((0, 64), dtype=torch.int8, device=DEV), torch.empty(0, device=DEV),
                     torch.zeros((5, 16), dtype=torch.uint8, device=DEV), torch.zeros(1, device=DEV), y)
    y2 = torch.full((3, 0), 1.0, device=DEV)
    tw.bitnet_linear(torch.zeros((3, 64), dtype=torch.int8, device=DEV), torch.zeros(3, device=DEV),
                     torch.zeros((0, 16), dtype=torch.uint8, device=DEV), torch.zeros(1, device=DEV), y2)
    # the same for the other entry points: nothing is launched, nothing is written
    q, s = tw.swiglu_quant(torch.empty((0, 64), device=DEV), torch.empty((0, 64), device=DEV))
    assert q.shape == (0, 64) and s.shape == (0,)
    q, s = tw.rmsnorm_quant(torch.empty((0, 64), dtype=torch.bfloat16, device=DEV), torch.ones(64, device=DEV), 1e-6)
    for fmt, wb in ((tw.FMT_BINARY, torch.zeros((5, 16), dtype=torch.uint8, device=DEV)),
                    (tw.FMT_BITPLANES, torch.zeros((5, 4, 8), dtype=torch.uint8, device=DEV))):
        y3 = tw.linear_bits(torch.empty((0, 128), dtype=torch.int8, device=DEV), torch.empty(0, device=DEV), wb, fmt,
                            torch.zeros(1, device=DEV))
        assert y3.shape == (0, 5)
    planes = tw.pack_bitplanes(torch.zeros((0, 32), dtype=torch.uint8, device=DEV), 128)
    assert planes.shape == (0, 4, 8)
    bits, s_w = tw.pack_weights_binary(torch.empty((0, 128), device=DEV))
    torch.cuda.synchronize()
    assert bits.shape == (0, 16) and s_w.item() == 0.0


def test_determinism():
    key = synth.stream_key(306)
    for M, N, K in [(1, 2560, 2560), (8, 640, 6912), (300, 700, 2560)]:
        x, q, s = quantized_inputs(synth.stream_key(key, M), M, K)
        packed = synth.random_bytes(synth.stream_key(key, M, 1), N * K // 4).numpy().reshape(N, K // 4)
        y1, a1 = gpu_linear(q, s, packed, 0.3)
        y2, a2 = gpu_linear(q, s, packed, 0.3)
        assert np.array_equal(a1, a2) and np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


# ----------------------------------------------------------------- full path, small

def test_end_to_end_single_gemv():
    """M = 1, K = N = 2560: bf16 N(0,1) activations with 0.1% x20 outliers, N(0, 0.02)
    latent weights, eps 1e-5, seed 0 -- every stage on the GPU against the oracle."""
    x, w = W.single_gemv()
    p_ref, sw_ref = oracle.pack(w.numpy(), 1e-5)
    q_ref, sx_ref = oracle.quant_act(bits_np(x))
    acc_ref, y_ref = oracle.linear(q_ref, sx_ref, p_ref, sw_ref)
    p, sw = tw.pack_weights(w.to(DEV), 1e-5)
    q, sx = tw.quant_act(x.to(DEV))
    y, acc = tw.linear(q, sx, p, sw, want_acc=True)
    assert sw.item() == sw_ref and np.array_equal(p.cpu().numpy(), p_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref) and np.array_equal(sx.cpu().numpy(), sx_ref)
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert_y(y.cpu().numpy(), y_ref)


@pytest.mark.parametrize("M", [1, 2, 4, 8, 16, 32, 64])
def test_batched_decode_sweep(M):
    """K = 2560, N = 6912 with M tokens, through the automatic kernel choice."""
    x = W.sweep_activations(M)
    w = W.sweep_weights()
    p_ref, sw_ref = oracle.pack(w.numpy(), 1e-5)
    q_ref, sx_ref = oracle.quant_act(bits_np(x))
    acc_ref, y_ref = oracle.linear(q_ref, sx_ref, p_ref, sw_ref)
    p, sw = tw.pack_weights(w.to(DEV), 1e-5)
    q, sx = tw.quant_act(x.to(DEV))
    y, acc = tw.linear(q, sx, p, sw, want_acc=True)
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert_y(y.cpu().numpy(), y_ref)


def test_grouped_plan_builders_check_tensors():
    """Wrong dtype, shape or a missing scale in any problem of a grouped plan is a
    ValueError raised before the C planner sees the pointers."""
    M, N, K = 1, 64, 256
    z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=DEV)
    q, sx, p, sw, y, acc = (z((M, K), torch.int8), z((M,), torch.float32), z((N, K // 4), torch.uint8),
                            z((1,), torch.float32), z((M, N), torch.float32), z((M, N), torch.int32))
    good = (q, sx, p, sw, y, acc)
    tw.bitnet_grouped_plan_linear([good])
    tw.bitnet_grouped_plan_linear([(q, sx, p, sw, z((M, N), torch.bfloat16), acc, 0, z((N,), torch.float32))])
    bad_linear = [
        (z((M, K), torch.uint8), sx, p, sw, y, acc),           # q dtype
        (q, z((2,), torch.float32), p, sw, y, acc),             # s_x shape
        (q, sx, z((N, K // 8), torch.uint8), sw, y, acc),       # packed shape
        (q, sx, p, z((2,), torch.float32), y, acc),             # s_w count
        (q, sx, p, sw, z((M, N + 1), torch.float32), acc),      # y shape
        (q, sx, p, sw, z((M, N), torch.float16), acc),          # y dtype (fp32 or bf16 only)
        (q, sx, p, sw, y, acc, 0, z((N + 1,), torch.float32)),  # bias shape
        (q, sx, p, sw, y, acc, 0, z((N,), torch.bfloat16)),     # bias dtype
        (q, sx, p, sw, y, z((M, N - 1), torch.int32)),          # acc shape
        (q, sx, p, sw, y, acc, 128),                            # w_group without N * K / 128 scales
    ]
    for i, prob in enumerate(bad_linear):
        with pytest.raises(ValueError):
            tw.bitnet_grouped_plan_linear([good, prob])
        assert i >= 0
    x = z((M, K), torch.bfloat16)
    tw.bitnet_grouped_plan_quant([(x, q, sx)])
    for prob in [(x, z((M, K + 64), torch.int8), sx), (x, q, z((M, 1), torch.float32)),
                 (z((M, K), torch.float32), q, sx)]:
        with pytest.raises(ValueError):
            tw.bitnet_grouped_plan_quant([prob])
    tw.bitnet_grouped_plan_fused([(x, p, sw, y, acc, q, sx)])
    for prob in [(x, p, sw, z((M, N - 1), torch.float32), None, None, None),
                 (x, p, sw, y, z((M, N), torch.float32), None, None),
                 (x, p, sw, y, None, z((M, K - 64), torch.int8), None),
                 (x, p, sw, y, None, None, z((M + 1,), torch.float32)),
                 (x, z((N, K // 4 - 1), torch.uint8), sw, y, None, None, None),
                 (x, (p, z((N + 1, K // 4), torch.uint8)), (sw, sw), y, None, None, None),
                 (x, p, sw, y, None, None, None, z((K + 1,), torch.float32), 1e-6),
                 (x, p, sw, z((M, N), torch.float16), None, None, None),
                 (x, p, sw, y, None, None, None, None, 0.0, z((N - 1,), torch.float32))]:
        with pytest.raises(ValueError):
            tw.bitnet_grouped_plan_fused([prob])


@pytest.mark.parametrize("M", [2, 5, 8, 16])
def test_grouped_mfma_decode_packed_at_line_offsets(M):
    """Grouped MFMA decode with each matrix's packed rows starting 16 .. 112 bytes into a
    128-byte line (views into one buffer at those byte offsets): the kernel loads whole
    lines and shifts each 16-row block's window by the rows' offset, whose period is 1, 2,
    4 or 8 rows for these K (K / 4 = 640, 1728, 160, 16 bytes per row).  acc bit for bit,
    y to the bound."""
    shapes = [(300, 2560, 16), (257, 6912, 48), (70, 640, 64), (33, 64, 112), (129, 6912, 80)]
    probs, refs = [], []
    for i, (N, K, off) in enumerate(shapes):
        key = synth.stream_key(331, M, i)
        x, q, s = quantized_inputs(key, M, K)
        packed = synth.random_bytes(synth.stream_key(key, 1), N * K // 4).numpy().reshape(N, K // 4)
        s_w = np.float32(0.0057 * (i + 1))
        refs.append(oracle.linear(q, s, packed, s_w))
        buf = torch.zeros(N * K // 4 + 256, dtype=torch.uint8, device=DEV)
        assert buf.data_ptr() % 128 == 0
        view = buf[off:off + N * K // 4].view(N, K // 4)
        view.copy_(torch.from_numpy(packed))
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        acc = torch.full((M, N), -1, dtype=torch.int32, device=DEV)
        probs.append((torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV), view,
                      torch.tensor([s_w], dtype=torch.float32, device=DEV), y, acc))
    plan = tw.bitnet_grouped_plan_linear(probs)
    plan.launch()
    torch.cuda.synchronize()
    for (acc_ref, y_ref), pr in zip(refs, probs):
        assert np.array_equal(pr[5].cpu().numpy(), acc_ref)
        assert_y(pr[4].cpu().numpy(), y_ref)


@pytest.mark.parametrize("M,N,K", [(2, 131072 + 300, 128), (8, 131072 + 17, 704), (16, 131072, 256), (5, 140000, 6912 // 4)])
def test_linear_many_rows_line_granular(M, N, K):
    """bitnet_linear with 2..16 tokens on a matrix of 131072 rows or more runs the
    line-granular MFMA decode kernel (one 256-row block per workgroup); ragged last
    block, rows starting mid-line (K / 4 = 32, 176, 64, 432 bytes per row)."""
    key = synth.stream_key(332, M, N, K)
    x, q, s = quantized_inputs(key, M, K)
    packed = synth.random_bytes(synth.stream_key(key, 1), N * K // 4).numpy().reshape(N, K // 4)
    check_linear(q, s, packed, np.float32(0.0043), kernels=(0, 4))


@pytest.mark.parametrize("M", [2, 7, 16])
def test_grouped_mfma_decode_groups_across_windows(M):
    """Group-wise scales on the line-granular MFMA decode kernel with groups longer than a
    step's 8 chunks (G = 640 and 1728: 10 and 27 chunks), K long enough for several staged
    segments (K = 30720, G = 3840), rows starting mid-line (K = 6912), a bias on some
    problems: acc bit for bit, y within the group-wise bound."""
    shapes = [(300, 2560, 640, False), (257, 6912, 1728, True), (70, 30720, 3840, False), (129, 6912, 64, True)]
    probs, refs = [], []
    for i, (N, K, G, with_bias) in enumerate(shapes):
        key = synth.stream_key(333, M, i)
        x, q, s = quantized_inputs(key, M, K)
        w = synth.latent_weights(synth.stream_key(key, 1), N, K, 0.02).numpy()
        w[:, :G] *= 3.0
        packed, s_w = oracle.pack_grouped(w, G, 1e-5)
        bias = _bias(key, N) if with_bias else None
        acc_ref, y_ref = oracle.linear_grouped(q, s, packed, s_w, G, bias)
        refs.append((acc_ref, y_ref, _grouped_bound(q, s, packed, s_w, G, K)))
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        acc = torch.full((M, N), -1, dtype=torch.int32, device=DEV)
        probs.append((torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV), torch.from_numpy(packed).to(DEV),
                      torch.from_numpy(s_w).to(DEV), y, acc, G,
                      None if bias is None else torch.from_numpy(bias).to(DEV)))
    plan = tw.bitnet_grouped_plan_linear(probs)
    for _ in range(2):
        plan.launch()
        torch.cuda.synchronize()
        for i, ((acc_ref, y_ref, slack), pr) in enumerate(zip(refs, probs)):
            assert np.array_equal(pr[5].cpu().numpy(), acc_ref), i
            assert_y_within(pr[4].cpu().numpy(), y_ref, REL, slack)


def test_grouped_plan_variant_reported():
    """GroupedPlan.variant reads the kernel choice from the plan header: the GEMV for
    one token, the line-granular MFMA decode kernel for several, its group-wise path
    when a problem has group-wise weight scales (nothing is launched)."""
    def plan(M, group):
        K, N = 256, 64
        q = torch.zeros((M, K), dtype=torch.int8, device=DEV)
        sx = torch.ones(M, dtype=torch.float32, device=DEV)
        p = torch.zeros((N, K // 4), dtype=torch.uint8, device=DEV)
        sw = torch.ones((N, K // group) if group else 1, dtype=torch.float32, device=DEV)
        y = torch.empty((M, N), dtype=torch.float32, device=DEV)
        return tw.bitnet_grouped_plan_linear([(q, sx, p, sw, y, None, group)])
    assert plan(1, 0).variant == 0
    assert plan(8, 0).variant == 1
    assert plan(8, 128).variant == 4
