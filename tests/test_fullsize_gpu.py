"""Full-size workloads on the GPU, in the launch configuration the bench times,
checked against the CPU oracle on sampled matrices / rows / columns.

* decode step: 30 layers x {q, k, v, o, gate, up, down} of the 2.4B shape:
  one grouped quant launch + one grouped linear launch at M = 1 and M = 8, the
  one fused launch at M = 1, and the fused launch with RMSNorm, without and with
  SwiGLU at both ends of the feed-forward part (layers 0 and 29 compared in
  full, every output checked for finiteness);
* prefill: M = 2048 on up (2560 -> 6912) and down (6912 -> 2560), natural
  density and 30 / 50 / 70 % nonzero codes, 160 sampled output columns;
* prefill as timed (y only, and bias + bf16 y) on 96 sampled token rows, and
  with group-128 weight scales on 64 sampled rows;
* 100B-scale FFN: gate (8192 -> 28672) and down (28672 -> 8192) of layer 0 at
  M = 1 and M = 8, compared in full; the 8-layer grouped launch as timed, its
  last layer compared in full;
* sign / mask bitplanes and binary weights at the stacked 229376 x 8192 shape,
  3 sampled row slices;
* the decode step with group-128 weight scales (grouped quant + grouped GEMV).
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import workloads as W
import ternary_weight_token_amd as tw

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REL = 2.0 ** -23


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    tw.lib()
    oracle.set_threads(min(16, max(1, len(os.sched_getaffinity(0)))))


def bits_np(x):
    return synth.bf16_bits(x.contiguous().cpu()).numpy().view(np.uint16)


def assert_y(y, y_ref):
    """fp32 y bit for bit: library and oracle both form acc * ((s_x s_w) / 127) in
    float64 and round once."""
    assert np.array_equal(np.ascontiguousarray(y, dtype=np.float32).view(np.uint32),
                          np.ascontiguousarray(y_ref, dtype=np.float32).view(np.uint32))


def swiglu_pair_bound(y_g, y_u, rel):
    """How far a = silu(g) u can move when g and u each move by rel of themselves,
    plus one fp32 rounding of a."""
    g = y_g.astype(np.float64)
    u = y_u.astype(np.float64)
    sg = 1.0 / (1.0 + np.exp(-g))
    dsilu = sg * (1.0 + g * (1.0 - sg))
    a = g * sg * u
    return 2 * rel * (np.abs(dsilu * g * u) + np.abs(a)) + 2.0 ** -23 * np.abs(a)


@pytest.mark.parametrize("M", [1, 8])
def test_decode_step_grouped(M):
    """The 30-layer decode step as one grouped quant launch and one grouped linear
    launch (the GEMV at M = 1, the MFMA decode kernel at M = 8): layers 0 and 29
    compared in full, every output finite."""
    mats = W.decode_step_2p4b(30)
    sample = {0, 29}
    packed, sws, host_w = [], [], {}
    for i, m in enumerate(mats):
        w = W.weights(m, DEV)
        p, s = tw.pack_weights(w, 1e-5)
        packed.append(p)
        sws.append(s)
        if m.layer in sample:
            host_w[i] = w.cpu()
        del w
    xs = [W.decode_step_activations(l, DEV, M) for l in range(30)]
    qs = [[torch.empty((M, x.shape[1]), dtype=torch.int8, device=DEV) for x in xl] for xl in xs]
    sxs = [[torch.empty(M, dtype=torch.float32, device=DEV) for _ in xl] for xl in xs]
    qplan = tw.bitnet_grouped_plan_quant(
        [(xs[l][s], qs[l][s], sxs[l][s]) for l in range(30) for s in range(4)])
    ys, accs, probs = [], [], []
    for i, m in enumerate(mats):
        y = torch.full((M, m.N), float("nan"), dtype=torch.float32, device=DEV)
        acc = torch.empty((M, m.N), dtype=torch.int32, device=DEV) if m.layer in sample else None
        ys.append(y)
        accs.append(acc)
        probs.append((qs[m.layer][m.slot], sxs[m.layer][m.slot], packed[i], sws[i], y, acc))
    lplan = tw.bitnet_grouped_plan_linear(probs)
    qplan.launch()
    for _ in range(4):   # repeated launches of one plan (the work counters reset each time)
        lplan.launch()
    torch.cuda.synchronize()
    for y in ys:
        y.fill_(float("nan"))
    lplan.launch()
    torch.cuda.synchronize()
    for y in ys:
        assert torch.isfinite(y).all()
    for l in sorted(sample):
        for s in range(4):
            q_ref, sx_ref = oracle.quant_act(bits_np(xs[l][s]))
            assert np.array_equal(qs[l][s].cpu().numpy(), q_ref)
            assert np.array_equal(sxs[l][s].cpu().numpy(), sx_ref)
    for i, m in enumerate(mats):
        if m.layer not in sample:
            continue
        p_ref, sw_ref = oracle.pack(host_w[i].numpy(), 1e-5)
        assert sws[i].item() == sw_ref
        assert np.array_equal(packed[i].cpu().numpy(), p_ref)
        q_ref, sx_ref = oracle.quant_act(bits_np(xs[m.layer][m.slot]))
        acc_ref, y_ref = oracle.linear(q_ref, sx_ref, p_ref, sw_ref)
        assert np.array_equal(accs[i].cpu().numpy(), acc_ref), (m.layer, m.name)
        assert_y(ys[i].cpu().numpy(), y_ref)


def test_decode_step_fused():
    """The 30-layer decode step as one fused launch (quantization inside the GEMV):
    layers 0 and 29 compared in full (q, s_x, acc, y), every other output finite."""
    mats = W.decode_step_2p4b(30)
    sample = {0, 29}
    xs = [W.decode_step_activations(l, DEV) for l in range(30)]
    probs, host = [], {}
    for i, m in enumerate(mats):
        w = W.weights(m, DEV)
        p, s = tw.pack_weights(w, 1e-5)
        if m.layer in sample:
            host[i] = w.cpu()
        del w
        y = torch.full((1, m.N), float("nan"), dtype=torch.float32, device=DEV)
        acc = torch.empty((1, m.N), dtype=torch.int32, device=DEV) if m.layer in sample else None
        q = torch.empty((1, m.K), dtype=torch.int8, device=DEV) if m.layer in sample else None
        sx = torch.empty(1, dtype=torch.float32, device=DEV) if m.layer in sample else None
        probs.append((xs[m.layer][m.slot], p, s, y, acc, q, sx))
    plan = tw.bitnet_grouped_plan_fused(probs)
    plan.launch()
    torch.cuda.synchronize()
    for pr in probs:
        assert torch.isfinite(pr[3]).all()
    for i, m in enumerate(mats):
        if m.layer not in sample:
            continue
        p_ref, sw_ref = oracle.pack(host[i].numpy(), 1e-5)
        q_ref, sx_ref = oracle.quant_act(bits_np(xs[m.layer][m.slot]))
        acc_ref, y_ref = oracle.linear(q_ref, sx_ref, p_ref, sw_ref)
        x, p, s, y, acc, q, sx = probs[i]
        assert np.array_equal(q.cpu().numpy(), q_ref) and np.array_equal(sx.cpu().numpy(), sx_ref)
        assert np.array_equal(acc.cpu().numpy(), acc_ref), (m.layer, m.name)
        assert_y(y.cpu().numpy(), y_ref)


@pytest.mark.parametrize("swiglu", [False, True])
def test_decode_step_fused_rmsnorm_swiglu(swiglu):
    """The 30-layer decode step as the one fused launch with RMSNorm before q / k / v
    and gate / up; with swiglu, each layer's gate / up as one pair problem whose
    epilogue writes a = fp32(silu(y_gate) y_up) and down taking an fp32 row: layers
    0 and 29 compared in full against the oracle (pairs bit for bit, codes and acc
    exactly, normed y within 2^-22 |y|), every output finite."""
    mats = W.decode_step_2p4b(30)
    sample = {0, 29}
    xs = [W.decode_step_activations(l, DEV) for l in range(30)]
    gains = [W.decode_step_gains(l, DEV) for l in range(30)]
    hidden = [W.decode_step_ffn_hidden(l, DEV) for l in range(30)]
    packed, sws, host = [], [], {}
    for i, m in enumerate(mats):
        w = W.weights(m, DEV)
        p, s = tw.pack_weights(w, 1e-5)
        packed.append(p)
        sws.append(s)
        if m.layer in sample:
            host[i] = w.cpu()
        del w
    probs, cases = [], []
    for i, m in enumerate(mats):
        if swiglu and m.name == "up":
            continue
        if swiglu and m.name == "gate":
            iu = next(j for j, o in enumerate(mats) if o.layer == m.layer and o.name == "up")
            y = torch.full((1, m.N), float("nan"), dtype=torch.float32, device=DEV)
            probs.append((xs[m.layer][m.slot], (packed[i], packed[iu]), (sws[i], sws[iu]), y, None, None, None,
                          gains[m.layer].get(m.slot), 1e-6))
            cases.append((m, "pair", (i, iu)))
            continue
        acc = torch.empty((1, m.N), dtype=torch.int32, device=DEV) if m.layer in sample else None
        y = torch.full((1, m.N), float("nan"), dtype=torch.float32, device=DEV)
        if swiglu and m.slot == W.SWIGLU_SLOT_2P4B:
            probs.append((hidden[m.layer], packed[i], sws[i], y, acc, None, None))
            cases.append((m, "f32", (i,)))
        else:
            gn = gains[m.layer].get(m.slot)
            probs.append((xs[m.layer][m.slot], packed[i], sws[i], y, acc, None, None, gn, 1e-6))
            cases.append((m, "plain" if gn is None else "norm", (i,)))
    plan = tw.bitnet_grouped_plan_fused(probs)
    plan.launch()
    torch.cuda.synchronize()
    for pr in probs:
        assert torch.isfinite(pr[3]).all()
    for pr, (m, kind, idx) in zip(probs, cases):
        if m.layer not in sample:
            continue
        refs = [oracle.pack(host[j].numpy(), 1e-5) for j in idx]
        if kind == "f32":
            q_ref, sx_ref = oracle.quant_act_f32(hidden[m.layer].cpu().numpy())
        elif kind == "plain":
            q_ref, sx_ref = oracle.quant_act(bits_np(xs[m.layer][m.slot]))
        else:
            gn = gains[m.layer][m.slot].cpu().numpy()
            q_ref, sx_ref = oracle.rmsnorm_quant(bits_np(xs[m.layer][m.slot]), gn, 1e-6)
        y = pr[3].cpu().numpy()
        if kind == "pair":
            (pg, sg), (pu, su) = refs
            _, y_g = oracle.linear(q_ref, sx_ref, pg, sg)
            _, y_u = oracle.linear(q_ref, sx_ref, pu, su)
            a_ref = oracle.swiglu_quant(y_g, y_u)[0]
            if gains[m.layer].get(m.slot) is None:
                assert np.array_equal(y, a_ref), (m.layer, m.name)
            else:
                # RMSNorm rows: s_x within one fp32 unit of the oracle's
                bound = swiglu_pair_bound(y_g, y_u, 2.0 ** -22)
                assert np.all(np.abs(y.astype(np.float64) - a_ref.astype(np.float64)) <= bound), (m.layer, m.name)
            continue
        (p_ref, sw_ref), = refs
        acc_ref, y_ref = oracle.linear(q_ref, sx_ref, p_ref, sw_ref)
        assert np.array_equal(pr[4].cpu().numpy(), acc_ref), (m.layer, m.name)
        if kind == "norm":
            d = np.abs(y.astype(np.float64) - y_ref.astype(np.float64))
            assert np.all(d <= 2.0 ** -22 * np.abs(y_ref.astype(np.float64))), (m.layer, m.name)
        else:
            assert_y(y, y_ref)


@pytest.mark.parametrize("name", ["up", "down"])
@pytest.mark.parametrize("density", [None, 0.3, 0.5, 0.7])
def test_prefill_sampled(name, density):
    x, w = W.prefill_inputs(name, density)
    N, K = w.shape
    p_ref, sw_ref = oracle.pack(w.numpy(), 1e-5)
    q_ref, sx_ref = oracle.quant_act(bits_np(x))
    p, sw = tw.pack_weights(w.to(DEV), 1e-5)
    q, sx = tw.quant_act(x.to(DEV))
    y, acc = tw.linear(q, sx, p, sw, want_acc=True)
    torch.cuda.synchronize()
    assert sw.item() == sw_ref and np.array_equal(p.cpu().numpy(), p_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref) and np.array_equal(sx.cpu().numpy(), sx_ref)
    cols = np.sort(np.random.default_rng(7).choice(N, 160, replace=False))
    cols[-1] = N - 1
    acc_ref, y_ref = oracle.linear(q_ref, sx_ref, np.ascontiguousarray(p_ref[cols]), sw_ref)
    assert np.array_equal(acc.cpu().numpy()[:, cols], acc_ref)
    assert_y(y.cpu().numpy()[:, cols], y_ref)


@pytest.mark.parametrize("name", ["up", "down"])
def test_prefill_timed_form(name):
    """The prefill GEMM exactly as timed: y only (no int32 accumulators requested,
    so the kernel takes its y-only store path), and the bias + bf16 form, at
    M = 2048 on the full N = 6912 / 2560; 96 sampled token rows (the first and
    last, and rows in every 128-row tile) compared over all N columns."""
    x, w = W.prefill_inputs(name, None)
    N, K = w.shape
    p_ref, sw_ref = oracle.pack(w.numpy(), 1e-5)
    q_ref, sx_ref = oracle.quant_act(bits_np(x))
    p, sw = tw.pack_weights(w.to(DEV), 1e-5)
    q, sx = tw.quant_act(x.to(DEV))
    y = torch.full((2048, N), float("nan"), dtype=torch.float32, device=DEV)
    tw.bitnet_linear(q, sx, p, sw, y)
    bias = torch.linspace(-1.0, 1.0, N, dtype=torch.float32)
    yb = tw.linear(q, sx, p, sw, bias=bias.to(DEV), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 2047], np.arange(16) * 128 + rng.integers(0, 128, 16),
                                     rng.choice(2048, 78, replace=False)]))
    qs = np.ascontiguousarray(q_ref[rows])
    _, y_ref = oracle.linear(qs, np.ascontiguousarray(sx_ref[rows]), p_ref, sw_ref)
    assert_y(y.cpu().numpy()[rows], y_ref)
    _, yb_ref = oracle.linear(qs, np.ascontiguousarray(sx_ref[rows]), p_ref, sw_ref, bias=bias.numpy())
    got = yb.cpu().view(torch.int16).numpy().view(np.uint16)[rows]
    assert np.array_equal(got, oracle.to_bf16(yb_ref))
    assert torch.isfinite(y).all()


def _gemm_group_bound(q, s_x, packed, s_w, G, K):
    """(K / G + 1) 2^-24 (s_x / 127) sum_g |acc_g s_g|: one rounding of each scaled
    group sum and of each running fp32 sum."""
    t = oracle.unpack(packed, K).astype(np.float64)
    qf = q.astype(np.float64)
    mag = np.zeros((q.shape[0], t.shape[0]))
    for g in range(K // G):
        sl = slice(g * G, (g + 1) * G)
        mag += np.abs(qf[:, sl] @ t[:, sl].T) * s_w[:, g].astype(np.float64)[None, :]
    return (K // G + 1) * 2.0 ** -24 * mag * (s_x.astype(np.float64)[:, None] / 127.0)


@pytest.mark.parametrize("name", ["up", "down"])
def test_prefill_group128_scales(name):
    """Prefill at M = 2048 with one weight scale per 128 weights (the pipelined GEMM's
    group-wise path, y only, as timed): 64 sampled token rows over all N columns,
    within the bound of its fp32 group accumulation."""
    x, w = W.prefill_inputs(name, None)
    N, K = w.shape
    p_ref, sw_ref = oracle.pack_grouped(w.numpy(), 128, 1e-5)
    q_ref, sx_ref = oracle.quant_act(bits_np(x))
    p, sw = tw.pack_weights_grouped(w.to(DEV), 128, 1e-5)
    q, sx = tw.quant_act(x.to(DEV))
    y = torch.full((2048, N), float("nan"), dtype=torch.float32, device=DEV)
    tw.bitnet_linear_ex(q, sx, p, sw, None, y, None, 0, w_group=128)
    torch.cuda.synchronize()
    assert np.array_equal(p.cpu().numpy(), p_ref) and np.array_equal(sw.cpu().numpy(), sw_ref)
    rows = np.unique(np.concatenate([[0, 2047], np.random.default_rng(13).choice(2048, 62, replace=False)]))
    qs, ss = np.ascontiguousarray(q_ref[rows]), np.ascontiguousarray(sx_ref[rows])
    _, y_ref = oracle.linear_grouped(qs, ss, p_ref, sw_ref, 128)
    slack = _gemm_group_bound(qs, ss, p_ref, sw_ref, 128, K)
    d = np.abs(y.cpu().numpy()[rows].astype(np.float64) - y_ref.astype(np.float64))
    assert not (d > REL * np.abs(y_ref.astype(np.float64)) + slack).any()
    assert torch.isfinite(y).all()


def test_ffn_100b_grouped_timed_form():
    """The 100B-scale FFN stream exactly as timed: 8 layers x {gate, up, down} in one
    grouped launch at M = 1 (the decode GEMV) and M = 8 (the MFMA decode kernel);
    the last layer's three matrices compared in full, every output finite."""
    mats = W.ffn_100b(8)
    sample = 7
    packed, sws, host_w = [], [], {}
    for i, m in enumerate(mats):
        w = W.weights(m, DEV)
        p, s = tw.pack_weights(w, 1e-5)
        packed.append(p)
        sws.append(s)
        if m.layer == sample:
            host_w[i] = w.cpu().numpy()
        del w
    refs = {i: oracle.pack(wh, 1e-5) for i, wh in host_w.items()}
    host_w.clear()
    for M in (1, 8):
        xs = [W.ffn_100b_activations(l, M, DEV) for l in range(8)]
        qx = [[tw.quant_act(x) for x in xl] for xl in xs]
        ys = [torch.full((M, m.N), float("nan"), dtype=torch.float32, device=DEV) for m in mats]
        accs = [torch.empty((M, m.N), dtype=torch.int32, device=DEV) if m.layer == sample else None for m in mats]
        plan = tw.bitnet_grouped_plan_linear(
            [(qx[m.layer][m.slot][0], qx[m.layer][m.slot][1], packed[i], sws[i], ys[i], accs[i])
             for i, m in enumerate(mats)])
        plan.launch()
        torch.cuda.synchronize()
        for y in ys:
            assert torch.isfinite(y).all()
        for i, (p_ref, sw_ref) in refs.items():
            m = mats[i]
            assert sws[i].item() == sw_ref
            q_ref, sx_ref = oracle.quant_act(bits_np(xs[m.layer][m.slot]))
            acc_ref, y_ref = oracle.linear(q_ref, sx_ref, p_ref, sw_ref)
            assert np.array_equal(accs[i].cpu().numpy(), acc_ref), (M, m.name)
            assert_y(ys[i].cpu().numpy(), y_ref)
        del xs, qx, ys, accs, plan


@pytest.mark.parametrize("which", [0, 2])  # gate (8192 -> 28672), down (28672 -> 8192)
def test_ffn_100b_layer0(which):
    m = W.ffn_100b(1)[which]
    w = W.weights(m, DEV)
    p, sw = tw.pack_weights(w, 1e-5)
    w_host = w.cpu().numpy()
    del w
    p_ref, sw_ref = oracle.pack(w_host, 1e-5)
    assert sw.item() == sw_ref
    assert np.array_equal(p.cpu().numpy(), p_ref)
    for M in (1, 8):
        x = W.ffn_100b_activations(0, M)[m.slot]
        q, sx = tw.quant_act(x.to(DEV))
        y, acc = tw.linear(q, sx, p, sw, want_acc=True)
        q_ref, sx_ref = oracle.quant_act(bits_np(x))
        acc_ref, y_ref = oracle.linear(q_ref, sx_ref, p_ref, sw_ref)
        assert np.array_equal(acc.cpu().numpy(), acc_ref)
        assert_y(y.cpu().numpy(), y_ref)


def test_bitplanes_stacked_100b_gate():
    """Sign / mask bitplanes at the encodings leg's one-launch shape (the 8 gate
    matrices of the 100B-scale FFN stacked: N = 229376, K = 8192, M = 1, the 4-row
    tile of the bit-serial GEMV): planes packed on the GPU and y / acc of three
    sampled 512-row slices (first, middle, last) against the oracle, every y finite."""
    N, K = 229376, 8192
    key = synth.stream_key(361, N, K)
    packed = synth.random_bytes(key, N * K // 4, DEV).view(N, K // 4)
    planes = tw.pack_bitplanes(packed, K)
    x = synth.activations(synth.stream_key(key, 1), 1, K, outlier_frac=0.001)
    q_ref, s_ref = oracle.quant_act(bits_np(x))
    q, sx = torch.from_numpy(q_ref).to(DEV), torch.from_numpy(s_ref).to(DEV)
    s_w = np.float32(0.0117)
    y, acc = tw.linear_bits(q, sx, planes, tw.FMT_BITPLANES, torch.tensor([s_w], device=DEV), want_acc=True)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    for r0 in (0, N // 2 - 256, N - 512):
        rows = slice(r0, r0 + 512)
        p_np = packed[rows].cpu().numpy()
        pl_ref = oracle.pack_bitplanes(p_np, K)
        assert np.array_equal(planes[rows].cpu().numpy(), pl_ref), r0
        acc_ref, y_ref = oracle.linear_bitplanes(q_ref, s_ref, pl_ref, s_w)
        assert np.array_equal(acc[:, rows].cpu().numpy(), acc_ref), r0
        assert_y(y[:, rows].cpu().numpy(), y_ref)


def test_binary_stacked_100b_gate():
    """b1.0 binary weights at the same stacked shape (N = 229376, K = 8192, M = 1):
    random weight bits (every pattern is a valid set of +1 / -1 weights), y / acc of
    three sampled 512-row slices against the oracle, every y finite."""
    N, K = 229376, 8192
    key = synth.stream_key(362, N, K)
    bits = synth.random_bytes(key, N * K // 8, DEV).view(N, K // 8)
    x = synth.activations(synth.stream_key(key, 1), 1, K, outlier_frac=0.001)
    q_ref, s_ref = oracle.quant_act(bits_np(x))
    q, sx = torch.from_numpy(q_ref).to(DEV), torch.from_numpy(s_ref).to(DEV)
    s_w = np.float32(0.0093)
    y, acc = tw.linear_bits(q, sx, bits, tw.FMT_BINARY, torch.tensor([s_w], device=DEV), want_acc=True)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    for r0 in (0, N // 2 - 256, N - 512):
        rows = slice(r0, r0 + 512)
        acc_ref, y_ref = oracle.linear_binary(q_ref, s_ref, bits[rows].cpu().numpy(), s_w, K)
        assert np.array_equal(acc[:, rows].cpu().numpy(), acc_ref), r0
        assert_y(y[:, rows].cpu().numpy(), y_ref)


def _grouped_bound(q, s_x, packed, s_w, G, K):
    """2^-44 (s_x / 127) sum_g |acc_g s_g| per output: the library sums the groups'
    float64 terms in another order than the oracle."""
    t = oracle.unpack(packed, K).astype(np.float64)
    sg = np.repeat(s_w.astype(np.float64), G, axis=1)
    mag = np.abs(q.astype(np.float64)) @ (np.abs(t) * sg).T
    return 2.0 ** -44 * mag * (s_x.astype(np.float64)[:, None] / 127.0)


def test_decode_step_grouped_group128_scales():
    """The 30-layer decode step with a weight scale per group of 128 weights, as
    one grouped quant launch and one grouped linear launch: layers 0 and 29 (packed
    bytes, scales, acc and y) against the oracle, every output finite."""
    G = 128
    mats = W.decode_step_2p4b(30)
    sample = {0, 29}
    xs = [W.decode_step_activations(l, DEV) for l in range(30)]
    qs = [[torch.empty((1, x.shape[1]), dtype=torch.int8, device=DEV) for x in xl] for xl in xs]
    sxs = [[torch.empty(1, dtype=torch.float32, device=DEV) for _ in xl] for xl in xs]
    qplan = tw.bitnet_grouped_plan_quant([(xs[l][j], qs[l][j], sxs[l][j]) for l in range(30) for j in range(4)])
    probs, host = [], {}
    for i, m in enumerate(mats):
        w = W.weights(m, DEV)
        p, sw = tw.pack_weights_grouped(w, G, 1e-5)
        if m.layer in sample:
            host[i] = w.cpu()
        del w
        y = torch.full((1, m.N), float("nan"), dtype=torch.float32, device=DEV)
        acc = torch.empty((1, m.N), dtype=torch.int32, device=DEV) if m.layer in sample else None
        probs.append((qs[m.layer][m.slot], sxs[m.layer][m.slot], p, sw, y, acc, G))
    plan = tw.bitnet_grouped_plan_linear(probs)
    qplan.launch()
    plan.launch()
    torch.cuda.synchronize()
    for pr in probs:
        assert torch.isfinite(pr[4]).all()
    for i, m in enumerate(mats):
        if m.layer not in sample:
            continue
        p_ref, s_ref = oracle.pack_grouped(host[i].numpy(), G, 1e-5)
        _, _, p, sw, y, acc, _ = probs[i]
        assert np.array_equal(p.cpu().numpy(), p_ref) and np.array_equal(sw.cpu().numpy(), s_ref), (m.layer, m.name)
        q_ref, sx_ref = oracle.quant_act(bits_np(xs[m.layer][m.slot]))
        acc_ref, y_ref = oracle.linear_grouped(q_ref, sx_ref, p_ref, s_ref, G)
        assert np.array_equal(acc.cpu().numpy(), acc_ref), (m.layer, m.name)
        d = np.abs(y.cpu().numpy().astype(np.float64) - y_ref.astype(np.float64))
        bound = REL * np.abs(y_ref.astype(np.float64)) + _grouped_bound(q_ref, sx_ref, p_ref, s_ref, G, m.K)
        assert np.all(d <= bound), (m.layer, m.name)

