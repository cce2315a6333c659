"""Pins for the CPU oracle: checks against values and facts that do not come
from the oracle itself (hand-worked examples, exact rational arithmetic, brute
force, closed forms, library routines and invariants).

Definitions pinned (pages: "BitNet 深度拆解……" on chenxutan.com, sec. 2.2
absmean/absmax quantization, sec. 2.3 rescale, sec. 3.1 BitLinear.forward,
sec. 3.3 INT2 packing; "1-bit推理框架bitnet.cpp实测……" on 0539edu.com,
sec. 2.1 RoundClip).
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- helpers

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Exact conversion for values already representable in bf16."""
    a = np.asarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_fraction_to_f32(fr: Fraction) -> float:
    """Correct round-to-nearest-even of an exact rational to binary32 (normal range)."""
    if fr == 0:
        return 0.0
    sign = -1.0 if fr < 0 else 1.0
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length() - 23
    while a / Fraction(2) ** e >= 2 ** 24:
        e += 1
    while a / Fraction(2) ** e < 2 ** 23:
        e -= 1
    m = a / Fraction(2) ** e
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * math.ldexp(float(fl), e)


def assert_rescale_rounding(y, exact: Fraction, delta: Fraction, where=None):
    """The oracle's y = fp32(v), v = acc * c_m (+ b) formed in float64 with
    c_m = (s_x s_w) / 127, lies within delta of the exact value (float64 rounding
    of c_m, of the product and of the sum), so y is the correct rounding of some
    value in [exact - delta, exact + delta]: rounding is monotone, so y lies
    between the roundings of the two ends.  Away from an fp32 rounding boundary
    the two ends round alike and y is the correctly rounded exact value."""
    lo = round_fraction_to_f32(exact - delta)
    hi = round_fraction_to_f32(exact + delta)
    assert lo <= float(y) <= hi, (where, float(y), lo, hi)
    return lo == hi


def rne_int(num: np.ndarray, den: np.ndarray) -> np.ndarray:
    """Round-half-even of num/den for int64 arrays (den > 0), exact."""
    fl = np.floor_divide(num, den)
    rem = num - fl * den
    twice = 2 * rem
    up = (twice > den) | ((twice == den) & (fl % 2 != 0))
    return fl + up.astype(np.int64)


def decode_unpackbits(packed: np.ndarray, K: int) -> np.ndarray:
    """Independent decoder of the byte layout: numpy little-endian bit order,
    bit pairs (2i, 2i+1) -> code, weight = code - 1."""
    bits = np.unpackbits(packed.reshape(-1, 1), axis=1, bitorder="little")  # [B][8]
    codes = bits[:, 0::2].astype(np.int16) + 2 * bits[:, 1::2].astype(np.int16)  # [B][4]
    return (codes.reshape(packed.shape[0], K) - 1).astype(np.int8)


def parse_cases(name: str):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            out.append([p.strip() for p in line.split("|")])
    return out


# ----------------------------------------------------------------- generator

def test_splitmix64_published_first_output():
    # SplitMix64 seeded with 0: first output 0xE220A8397B1DCDAF (Vigna's
    # reference splitmix64.c), second 0x6E789E6AA1B965F4.
    assert synth.splitmix64_py(0, 2) == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4]


def test_generator_torch_matches_python():
    key = synth.stream_key(7, 3)
    ref = synth.splitmix64_py(key, 1000)
    got = synth.raw64(key, 0, 1000).tolist()
    assert [g & ((1 << 64) - 1) for g in got] == ref


def test_generator_normal_moments():
    z = synth.normal(synth.stream_key(1), 1 << 20)
    assert abs(z.mean().item()) < 5e-3
    assert abs(z.std().item() - 1.0) < 5e-3


# ----------------------------------------------------------------- pack

@pytest.mark.parametrize("case", parse_cases("pack_cases.txt"))
def test_pack_golden(case):
    eps = float(case[0])
    w = np.array([float(v) for v in case[1].split()], dtype=np.float32)[None, :]
    expect = np.array([int(b, 16) for b in case[2].split()], dtype=np.uint8)
    packed, s_w = oracle.pack(w, eps)
    assert packed[0].tolist() == expect.tolist()
    assert s_w == np.float32(float(case[3]))


def test_pack_layout_against_unpackbits():
    key = synth.stream_key(11)
    w = synth.density_weights(key, 37, 128, 0.6).numpy()
    t_expect = np.rint(w / 0.02).astype(np.int8)
    packed, _ = oracle.pack(w, 1e-5)
    assert np.array_equal(decode_unpackbits(packed, 128), t_expect)
    assert np.array_equal(oracle.unpack(packed, 128), t_expect)


def test_pack_all_zero_tensor():
    packed, s_w = oracle.pack(np.zeros((5, 64), np.float32), 1e-5)
    assert s_w == 0.0 and np.all(packed == 0x55)


def test_pack_sign_symmetry():
    w = synth.latent_weights(synth.stream_key(3), 64, 256, 0.02).numpy()
    p1, s1 = oracle.pack(w)
    p2, s2 = oracle.pack(-w)
    assert s1 == s2
    t1 = decode_unpackbits(p1, 256)
    t2 = decode_unpackbits(p2, 256)
    assert np.array_equal(t1, -t2)


def test_weight_scale_equals_exact_mean():
    # s_w must be the correctly rounded binary32 value of the exact mean of |W|.
    for seed in range(3):
        w = synth.latent_weights(synth.stream_key(4, seed), 48, 320, 0.02).numpy()
        s_w, rows = oracle.weight_scale(w)
        exact = sum(Fraction(float(v)) for v in np.abs(w).ravel()) / w.size
        assert s_w == np.float32(round_fraction_to_f32(exact))
        # row sums agree with exact row sums to float64 accuracy
        r0 = sum(Fraction(float(v)) for v in np.abs(w[0]))
        assert abs(Fraction(rows[0]) - r0) <= abs(r0) * Fraction(1, 2 ** 45)


def test_ternary_density_closed_form():
    # For w ~ N(0, s): mean|w| = s*sqrt(2/pi); t != 0 iff |w| > mean|w|/2, so
    # P(t != 0) = 2 * (1 - Phi(sqrt(2/pi)/2)) = 0.68996...
    w = synth.latent_weights(synth.stream_key(5), 2560, 2560, 0.02).numpy()
    packed, _ = oracle.pack(w, 1e-5)
    t = decode_unpackbits(packed, 2560)
    dens = float(np.count_nonzero(t)) / t.size
    c = math.sqrt(2 / math.pi) / 2
    expect = 2 * (1 - 0.5 * (1 + math.erf(c / math.sqrt(2))))
    assert abs(expect - 0.68996) < 1e-4
    assert abs(dens - expect) < 1.5e-3
    # and the latent scale: s_w ~ 0.02*sqrt(2/pi)
    s_w, _ = oracle.weight_scale(w)
    assert abs(float(s_w) / (0.02 * math.sqrt(2 / math.pi)) - 1) < 2e-3


def test_density_weights_round_trip():
    for d in (0.3, 0.5, 0.7):
        w = synth.density_weights(synth.stream_key(6, int(d * 10)), 64, 512, d).numpy()
        packed, s_w = oracle.pack(w, 1e-5)
        assert np.array_equal(decode_unpackbits(packed, 512), np.rint(w / 0.02).astype(np.int8))
        nz = np.count_nonzero(w)
        assert abs(float(s_w) - 0.02 * nz / w.size) < 1e-8


# ----------------------------------------------------------------- quant_act

@pytest.mark.parametrize("case", parse_cases("quant_act_cases.txt"))
def test_quant_golden(case):
    x = np.array([float(v) for v in case[0].split()], dtype=np.float32)[None, :]
    q, s = oracle.quant_act(f32_to_bf16_bits(x))
    assert q[0].tolist() == [int(v) for v in case[1].split()]
    assert s[0] == np.float32(float(case[2]))


def _exhaustive_rows(s_exp: int):
    """One row per bf16 s in the binade [2^s_exp, 2^(s_exp+1)); the row holds s
    followed by every bf16 x with |x| <= s over 13 binades below, both signs."""
    rows = []
    mant = np.arange(128, dtype=np.uint32)
    xs = []
    for e in range(s_exp - 12, s_exp + 1):
        xs.append(((e + 127) << 7) | mant)
    xs = np.concatenate(xs).astype(np.uint16)
    for m in range(128):
        s_bits = np.uint16(((s_exp + 127) << 7) | m)
        xv = xs[xs <= s_bits]
        row = np.concatenate([[s_bits], xv, xv | 0x8000]).astype(np.uint16)
        rows.append(row)
    width = max(len(r) for r in rows)
    # pad with +0 (does not change the max)
    out = np.zeros((len(rows), width), dtype=np.uint16)
    for i, r in enumerate(rows):
        out[i, :len(r)] = r
    return out


@pytest.mark.parametrize("s_exp", [0, -40, 50])
def test_quant_exhaustive_against_exact_rne(s_exp):
    x = _exhaustive_rows(s_exp)
    q, s = oracle.quant_act(x)
    # exact: x = mx * 2^ex, s = ms * 2^es (integers) -> 127*x/s rounded half-even
    xb = x.astype(np.int64)
    sign = np.where(xb & 0x8000, -1, 1)
    ex_field = (xb >> 7) & 0xFF
    mx = np.where(ex_field == 0, 0, (xb & 0x7F) | 0x80)
    sb = xb[:, :1]
    ms = (sb & 0x7F) | 0x80
    sh = ex_field - ((sb >> 7) & 0xFF)  # in [-12, 0] for nonzero x
    sh = np.where(mx == 0, 0, sh)
    num = 127 * mx * (1 << (sh + 12))
    den = ms * (1 << 12) * np.ones_like(num)
    expect = sign * rne_int(num, den)
    assert np.array_equal(q.astype(np.int64), expect)
    assert np.array_equal(s, bf16_bits_to_f32(x[:, 0]))
    # the same decision taken in binary32, (127*x)/s with one rounding each, is
    # identical: 127*x is exact for bf16 x, so the quotient has one rounding and
    # never lands on a tie it did not start on.
    xf = bf16_bits_to_f32(x)
    with np.errstate(divide="ignore", invalid="ignore"):
        q32 = np.rint((np.float32(127.0) * xf) / xf[:, :1]).astype(np.int64)
    assert np.array_equal(q32, expect)


def test_quant_invariants():
    x = synth.activations(synth.stream_key(8), 16, 512, outlier_frac=0.001)
    bits = synth.bf16_bits(x).numpy().view(np.uint16)
    q, s = oracle.quant_act(bits)
    # every nonzero row reaches +-127 exactly
    assert np.all(np.abs(q).max(axis=1) == 127)
    # x -> -x negates q and keeps s
    qn, sn = oracle.quant_act(bits ^ np.uint16(0x8000))
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    # x -> 2^j x keeps q, scales s by 2^j (exact in bf16)
    for j in (-7, 5):
        xs = (x.float() * (2.0 ** j)).to(torch.bfloat16)
        qj, sj = oracle.quant_act(synth.bf16_bits(xs).numpy().view(np.uint16))
        assert np.array_equal(qj, q)
        assert np.array_equal(sj, (s * np.float32(2.0 ** j)).astype(np.float32))


# ----------------------------------------------------------------- linear

def _brute_force(q, s_x, packed, s_w, K):
    """int64 triple loop in plain Python over decoded weights."""
    t = decode_unpackbits(packed, K).tolist()
    M = q.shape[0]
    N = packed.shape[0]
    acc = [[sum(int(q[m, k]) * t[n][k] for k in range(K)) for n in range(N)] for m in range(M)]
    return np.array(acc, dtype=np.int64)


@pytest.mark.parametrize("M,N,K", [(1, 1, 4), (3, 5, 8), (2, 7, 68), (5, 3, 132)])
def test_linear_brute_force(M, N, K):
    key = synth.stream_key(9, M, N, K)
    x = synth.activations(key, M, K)
    q, s = oracle.quant_act(synth.bf16_bits(x).numpy().view(np.uint16))
    packed = synth.random_bytes(synth.stream_key(key, 1), N * K // 4).numpy().reshape(N, K // 4)
    acc, y = oracle.linear(q, s, packed, np.float32(0.0137))
    assert np.array_equal(acc.astype(np.int64), _brute_force(q, s, packed, 0.0137, K))


def test_linear_matches_float64_matmul():
    key = synth.stream_key(10)
    M, N, K = 9, 300, 640
    x = synth.activations(key, M, K, outlier_frac=0.001)
    q, s = oracle.quant_act(synth.bf16_bits(x).numpy().view(np.uint16))
    w = synth.latent_weights(synth.stream_key(key, 5), N, K, 0.02).numpy()
    packed, s_w = oracle.pack(w)
    acc, y = oracle.linear(q, s, packed, s_w)
    t = decode_unpackbits(packed, K).astype(np.float64)
    ref = q.astype(np.float64) @ t.T
    assert np.array_equal(acc.astype(np.float64), ref)
    # and the rescale is a faithful approximation of the float model of the pages
    yref = ref * (s.astype(np.float64)[:, None] / 127.0) * float(s_w)
    assert np.allclose(y, yref, rtol=2 ** -23, atol=0)


def test_linear_k_permutation_invariance():
    key = synth.stream_key(12)
    M, N, K = 4, 33, 256
    x = synth.activations(key, M, K)
    q, s = oracle.quant_act(synth.bf16_bits(x).numpy().view(np.uint16))
    w = synth.density_weights(synth.stream_key(key, 1), N, K, 0.7).numpy()
    packed, s_w = oracle.pack(w)
    acc, y = oracle.linear(q, s, packed, s_w)
    perm = np.random.default_rng(0).permutation(K)
    packed_p, s_wp = oracle.pack(np.ascontiguousarray(w[:, perm]))
    assert s_wp == s_w
    acc_p, y_p = oracle.linear(np.ascontiguousarray(q[:, perm]), s, packed_p, s_w)
    assert np.array_equal(acc, acc_p) and np.array_equal(y, y_p)


def test_linear_negating_w_negates_outputs():
    key = synth.stream_key(13)
    M, N, K = 3, 50, 384
    x = synth.activations(key, M, K, outlier_frac=0.01)
    q, s = oracle.quant_act(synth.bf16_bits(x).numpy().view(np.uint16))
    w = synth.latent_weights(synth.stream_key(key, 1), N, K, 0.02).numpy()
    p1, s1 = oracle.pack(w)
    p2, s2 = oracle.pack(-w)
    a1, y1 = oracle.linear(q, s, p1, s1)
    a2, y2 = oracle.linear(q, s, p2, s2)
    assert np.array_equal(a1, -a2) and np.array_equal(y1, -y2)


def test_linear_all_plus_one_and_code3():
    key = synth.stream_key(14)
    M, N, K = 6, 4, 320
    x = synth.activations(key, M, K)
    q, s = oracle.quant_act(synth.bf16_bits(x).numpy().view(np.uint16))
    plus = np.full((N, K // 4), 0xAA, np.uint8)       # every code 2 -> +1
    acc, _ = oracle.linear(q, s, plus, np.float32(1.0))
    assert np.array_equal(acc, np.repeat(q.astype(np.int32).sum(1, keepdims=True), N, 1))
    three = np.full((N, K // 4), 0xFF, np.uint8)      # code 3 decodes to +2
    acc3, _ = oracle.linear(q, s, three, np.float32(1.0))
    assert np.array_equal(acc3, 2 * acc)
    zero = np.full((N, K // 4), 0x55, np.uint8)
    acc0, y0 = oracle.linear(q, s, zero, np.float32(0.5))
    assert np.all(acc0 == 0) and np.all(y0 == 0)
    # a constant positive row quantizes to 127 everywhere -> acc = 127 K
    xc = np.full((1, K), 0.75, np.float32)
    qc, sc = oracle.quant_act(f32_to_bf16_bits(xc))
    accc, _ = oracle.linear(qc, sc, plus[:1], np.float32(1.0))
    assert accc[0, 0] == 127 * K


# float64 error of acc * ((s_x s_w) / 127): s_x s_w is exact (48 significant bits), the
# quotient and the product are each rounded once, 2 * 2^-53 relative plus a product term
EPI_REL = Fraction(1, 2 ** 51)


def test_epilogue_rounding():
    """y against the exact rational acc s_x s_w / 127: the correctly rounded fp32
    value wherever the exact value is not within 2^-51 relative of a rounding
    boundary, which is every sampled output here."""
    key = synth.stream_key(15)
    M, N, K = 4, 200, 512
    x = synth.activations(key, M, K, row_scale=(0.1, 10.0))
    q, s = oracle.quant_act(synth.bf16_bits(x).numpy().view(np.uint16))
    w = synth.latent_weights(synth.stream_key(key, 1), N, K, 0.02).numpy()
    packed, s_w = oracle.pack(w)
    acc, y = oracle.linear(q, s, packed, s_w)
    decided = 0
    for m in range(M):
        for n in range(N):
            exact = Fraction(int(acc[m, n])) * Fraction(float(s[m])) * Fraction(float(s_w)) / 127
            decided += assert_rescale_rounding(y[m, n], exact, abs(exact) * EPI_REL, (m, n))
    assert decided == M * N      # every output here is the correctly rounded value
    # extreme accumulators
    qx = np.full((1, K), 127, np.int8)
    acc_x, y_x = oracle.linear(qx, np.array([3.0e5], np.float32), np.full((1, K // 4), 0xAA, np.uint8),
                               np.float32(7.77e-3))
    exact = Fraction(127 * K) * Fraction(float(np.float32(3.0e5))) * Fraction(float(np.float32(7.77e-3))) / 127
    assert assert_rescale_rounding(y_x[0, 0], exact, abs(exact) * EPI_REL)


def test_epilogue_one_factor_per_row():
    """The rescale is one float64 factor per token row, c_m = (s_x[m] s_w) / 127,
    times acc: scaling acc by 2^j (a power of two, exact) scales y by 2^j exactly,
    and two outputs of one row with acc and -acc are exact negatives."""
    K, N = 64, 4
    q = np.zeros((1, K), np.int8)
    q[0, 0], q[0, 1] = 100, 27
    packed = np.full((N, K // 4), 0x55, np.uint8)        # all codes 1 (weight 0)
    packed[0, 0] = 0x56                                 # weight +1 at k = 0
    packed[1, 0] = 0x54                                 # weight -1 at k = 0
    packed[2, 0] = 0x5A                                 # +1 at k = 0 and k = 1
    s = np.array([0.8317], np.float32)
    acc, y = oracle.linear(q, s, packed, np.float32(0.0137))
    assert list(acc[0]) == [100, -100, 127, 0]
    assert y[0, 0] == -y[0, 1] and y[0, 3] == 0.0
    c = (float(s[0]) * float(np.float32(0.0137))) / 127.0
    assert y[0, 0] == np.float32(100.0 * c) and y[0, 2] == np.float32(127.0 * c)


# ----------------------------------------------------------------- epilogue options

def _f32(bits: int) -> np.float32:
    return np.array([bits], np.uint32).view(np.float32)[0]


def test_to_bf16_hand_cases():
    # bf16 keeps 7 fraction bits: one unit in the last place at 1.0 is 2^-7
    cases = [
        (1.0, 0x3F80),
        (1.0 + 2.0 ** -8, 0x3F80),                 # tie, lower neighbour even
        (1.0 + 3 * 2.0 ** -8, 0x3F82),             # tie, lower neighbour odd -> up
        (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),    # just above the tie
        (-(1.0 + 3 * 2.0 ** -8), 0xBF82),
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (2.0 ** -133, 0x0001),                     # smallest bf16 subnormal
        (1.5 * 2.0 ** -133, 0x0002),               # tie between 1 (odd) and 2
        (2.0 ** -134, 0x0000),                     # tie between 0 (even) and 1
        (2.0 ** -149, 0x0000),                     # far below half the smallest
        (3.0e38, 0x7F62),                          # bf16 nearest to 3e38 below max
    ]
    vals = np.array([c[0] for c in cases], np.float32)
    got = oracle.to_bf16(vals)
    for (v, want), g in zip(cases, got):
        assert int(g) == want, (v, hex(int(g)), hex(want))
    # the largest finite fp32 lies above the midpoint to 2^128: overflow to +inf
    assert int(oracle.to_bf16(np.array([_f32(0x7F7FFFFF)]))[0]) == 0x7F80


def test_to_bf16_matches_torch_rounding():
    """The library conversion fp32 -> bfloat16 of torch (CPU) rounds to nearest even."""
    rng = np.random.default_rng(2024)
    hi = rng.integers(0, 1 << 16, size=1 << 18, dtype=np.uint32)
    parts = [rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)]
    for low in (0x8000, 0x7FFF, 0x8001, 0x0000, 0xFFFF):   # ties and their neighbours
        parts.append((hi << 16) | np.uint32(low))
    bits = np.concatenate(parts)
    bits = bits[((bits >> 23) & 0xFF) != 0xFF]             # finite inputs only
    f = bits.view(np.float32)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.to_bf16(f), want)


def test_to_bf16_is_nearest():
    """Every result is a bf16 value at distance <= half a unit from the input."""
    rng = np.random.default_rng(7)
    f = (rng.standard_normal(1 << 16) * np.exp2(rng.integers(-60, 60, 1 << 16))).astype(np.float32)
    b = oracle.to_bf16(f)
    back = bf16_bits_to_f32(b).astype(np.float64)
    e = np.floor(np.log2(np.maximum(np.abs(back), 1e-300)))
    half_ulp = np.exp2(e - 8)
    assert np.all(np.abs(back - f.astype(np.float64)) <= half_ulp * (1 + 1e-12))


@pytest.mark.parametrize("M,N,K", [(1, 3, 4), (3, 5, 8), (4, 7, 132)])
def test_linear_bias_exact(M, N, K):
    key = synth.stream_key(16, M, N, K)
    x = synth.activations(key, M, K, row_scale=(0.1, 10.0))
    q, s = oracle.quant_act(synth.bf16_bits(x).numpy().view(np.uint16))
    w = synth.latent_weights(synth.stream_key(key, 1), N, K, 0.02).numpy()
    packed, s_w = oracle.pack(w)
    bias = (np.arange(N, dtype=np.float32) - N / 2) * np.float32(0.37) + np.float32(0.011)
    acc, y = oracle.linear(q, s, packed, s_w, bias=bias)
    acc0, _ = oracle.linear(q, s, packed, s_w)
    assert np.array_equal(acc, acc0)                 # the bias leaves acc alone
    acc_bf = _brute_force(q, s, packed, s_w, K)
    for m in range(M):
        for n in range(N):
            prod = Fraction(int(acc_bf[m, n])) * Fraction(float(s[m])) * Fraction(float(s_w)) / 127
            exact = prod + Fraction(float(bias[n]))
            # float64: the product's error, then one rounding of the sum
            delta = abs(prod) * EPI_REL + abs(exact) * Fraction(1, 2 ** 52)
            assert assert_rescale_rounding(y[m, n], exact, delta, (m, n))


def test_linear_bias_broadcast_over_tokens():
    """A zero token row gives acc = 0, so every output of that row is the bias itself."""
    N, K = 9, 64
    q = np.zeros((3, K), np.int8)
    q[1] = 5
    s = np.array([0.0, 2.0, 0.0], np.float32)
    packed = synth.random_bytes(synth.stream_key(17), N * K // 4).numpy().reshape(N, K // 4)
    bias = np.linspace(-3, 3, N).astype(np.float32)
    _, y = oracle.linear(q, s, packed, np.float32(0.5), bias=bias)
    assert np.array_equal(y[0], bias) and np.array_equal(y[2], bias)
    assert not np.array_equal(y[1], bias)


# ----------------------------------------------------------------- RMSNorm + quantization

def _rms_scale_exact(z_max: Fraction, xs, eps: float) -> float:
    """fp32 of z_max / sqrt(mean(x^2) + eps), the square root to 60 digits."""
    import decimal
    ctx = decimal.Context(prec=60)
    ms = sum(Fraction(float(v)) ** 2 for v in xs) / len(xs) + Fraction(float(np.float32(eps)))
    d = ctx.sqrt(ctx.divide(decimal.Decimal(ms.numerator), decimal.Decimal(ms.denominator)))
    val = ctx.divide(decimal.Decimal(z_max.numerator), decimal.Decimal(z_max.denominator))
    return round_fraction_to_f32(Fraction(ctx.divide(val, d)))


def test_rmsnorm_quant_hand_case():
    x = f32_to_bf16_bits(np.array([[1.0, 2.0, 0.0, -1.0]], np.float32))
    q, s = oracle.rmsnorm_quant(x, np.ones(4, np.float32), 1e-6)
    # 127 z / max|z| = 63.5, 127, 0, -63.5: the halves go to the even neighbour
    assert q.tolist() == [[64, 127, 0, -64]]
    assert s[0] == np.float32(_rms_scale_exact(Fraction(2), [1.0, 2.0, 0.0, -1.0], 1e-6))


def test_rmsnorm_quant_unit_gain_is_plain_quantization():
    """With g = 1 the codes are those of the row itself (r cancels) and the scale is
    max|x| r."""
    key = synth.stream_key(20)
    x = synth.activations(key, 6, 640, outlier_frac=0.01, row_scale=(0.1, 10.0))
    bits = synth.bf16_bits(x).numpy().view(np.uint16)
    q0, s0 = oracle.quant_act(bits)
    q1, s1 = oracle.rmsnorm_quant(bits, np.ones(640, np.float32), 1e-5)
    assert np.array_equal(q0, q1)
    xf = bf16_bits_to_f32(bits)
    for m in range(6):
        assert s1[m] == np.float32(_rms_scale_exact(Fraction(float(s0[m])), xf[m].tolist(), 1e-5))


@pytest.mark.parametrize("K", [4, 68, 256])
def test_rmsnorm_quant_exact(K):
    """Codes against exact rational RNE of 127 x g / max|x g|; scale against the
    60-digit value of max|x g| / sqrt(mean(x^2) + eps)."""
    key = synth.stream_key(21, K)
    x = synth.activations(key, 5, K, outlier_frac=0.02)
    bits = synth.bf16_bits(x).numpy().view(np.uint16)
    g = (1.0 + 0.3 * synth.normal(synth.stream_key(key, 7), K).float().numpy()).astype(np.float32)
    g[::7] = -g[::7]
    eps = 1e-6
    q, s = oracle.rmsnorm_quant(bits, g, eps)
    xf = bf16_bits_to_f32(bits)
    for m in range(5):
        z = [Fraction(float(xf[m, k])) * Fraction(float(g[k])) for k in range(K)]
        zmax = max(abs(v) for v in z)
        for k in range(K):
            v = 127 * z[k] / zmax
            fl = v.numerator // v.denominator
            rem = v - fl
            r = fl + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2) else 0)
            assert q[m, k] == r, (m, k)
        assert s[m] == np.float32(_rms_scale_exact(zmax, xf[m].tolist(), eps)), m


def test_rmsnorm_quant_invariants():
    key = synth.stream_key(22)
    K = 512
    x = synth.activations(key, 4, K)
    bits = synth.bf16_bits(x).numpy().view(np.uint16)
    g = (0.5 + synth.uniform(synth.stream_key(key, 3), K, 0).float().numpy()).astype(np.float32)
    q, s = oracle.rmsnorm_quant(bits, g, 0.0)
    # x -> 2x (exact in bf16) with eps = 0 changes nothing, bit for bit
    x2 = f32_to_bf16_bits(bf16_bits_to_f32(bits) * np.float32(2.0))
    q2, s2 = oracle.rmsnorm_quant(x2, g, 0.0)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    # x -> -x negates the codes
    qn, sn = oracle.rmsnorm_quant(bits ^ np.uint16(0x8000), g, 0.0)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    # every row reaches 127 in magnitude
    assert np.all(np.abs(q).max(axis=1) == 127)
    # an all-zero row
    qz, sz = oracle.rmsnorm_quant(np.zeros((1, K), np.uint16), g, 1e-6)
    assert not qz.any() and sz[0] == 0.0


# ----------------------------------------------------------------- group-wise weight scales

def test_pack_grouped_hand_case():
    """Two groups of 4 in one row (eps = 0): group 0 = [0.5, -0.25, 0.1, 0] has
    mean |w| = 0.2125 and w / s = [2.35, -1.18, 0.47, 0] -> t = [1, -1, 0, 0] ->
    codes [2, 0, 1, 1] -> byte 0x52; group 1 = [2, 0.5, -0.5, 1] has mean 1 and
    w / s = [2, 0.5, -0.5, 1] -> t = [1, 0, 0, 1] (halves to even) -> byte 0x96."""
    w = np.array([[0.5, -0.25, 0.1, 0.0, 2.0, 0.5, -0.5, 1.0]], np.float32)
    packed, s_w = oracle.pack_grouped(w, 4, 0.0)
    assert packed.tolist() == [[0x52, 0x96]]
    assert s_w[0, 0] == np.float32(round_fraction_to_f32(
        (Fraction(0.5) + Fraction(0.25) + Fraction(float(np.float32(0.1)))) / 4))
    assert s_w[0, 1] == 1.0


def test_pack_per_channel_is_per_tensor_of_each_row():
    key = synth.stream_key(23)
    N, K = 7, 640
    w = synth.latent_weights(key, N, K, 0.02).numpy()
    w[3] *= 5.0
    packed, s_w = oracle.pack_grouped(w, K, 1e-5)
    for n in range(N):
        p_row, s_row = oracle.pack(np.ascontiguousarray(w[n:n + 1]), 1e-5)
        assert np.array_equal(packed[n:n + 1], p_row) and s_w[n, 0] == s_row


@pytest.mark.parametrize("G", [4, 128, 640])
def test_pack_grouped_scales_exact(G):
    key = synth.stream_key(24, G)
    N, K = 5, 640
    w = synth.latent_weights(key, N, K, 0.02).numpy()
    packed, s_w = oracle.pack_grouped(w, G, 1e-5)
    for n in range(N):
        for g in range(K // G):
            exact = sum(Fraction(float(abs(v))) for v in w[n, g * G:(g + 1) * G]) / G
            assert s_w[n, g] == np.float32(round_fraction_to_f32(exact))
    # each group's codes are the per-tensor codes of that group alone
    for n in (0, 4):
        for g in (0, K // G - 1):
            p_g, s_g = oracle.pack(np.ascontiguousarray(w[n:n + 1, g * G:(g + 1) * G]), 1e-5)
            assert s_g == s_w[n, g] and np.array_equal(p_g[0], packed[n, g * G // 4:(g + 1) * G // 4])


@pytest.mark.parametrize("M,N,K,G", [(1, 3, 256, 64), (3, 5, 512, 128), (2, 4, 384, 384)])
def test_linear_grouped_exact(M, N, K, G):
    key = synth.stream_key(25, M, N, K, G)
    x = synth.activations(key, M, K, row_scale=(0.1, 10.0))
    q, s = oracle.quant_act(synth.bf16_bits(x).numpy().view(np.uint16))
    w = synth.latent_weights(synth.stream_key(key, 1), N, K, 0.02).numpy()
    w[:, :G] *= 7.0                      # groups with very different scales
    packed, s_w = oracle.pack_grouped(w, G, 1e-5)
    bias = np.linspace(-1, 1, N).astype(np.float32)
    acc, y = oracle.linear_grouped(q, s, packed, s_w, G, bias=bias)
    t = decode_unpackbits(packed, K).astype(np.int64)
    for m in range(M):
        for n in range(N):
            groups = [int(np.dot(q[m, g * G:(g + 1) * G].astype(np.int64), t[n, g * G:(g + 1) * G]))
                      for g in range(K // G)]
            assert acc[m, n] == sum(groups)
            prod = (sum(Fraction(a) * Fraction(float(s_w[n, g])) for g, a in enumerate(groups))
                    * Fraction(float(s[m])) / 127)
            exact = prod + Fraction(float(bias[n]))
            if K // G == 1:
                # one scale per row: the per-tensor rescale with the row's own scale
                delta = abs(prod) * EPI_REL + abs(exact) * Fraction(1, 2 ** 52)
                assert assert_rescale_rounding(y[m, n], exact, delta, (m, n))
            else:
                assert y[m, n] == np.float32(round_fraction_to_f32(exact)), (m, n)


def test_linear_grouped_uniform_scales_match_per_tensor():
    """Every group with the same scale s: within one fp32 unit of the per-tensor form
    (the two associate the float64 products differently)."""
    key = synth.stream_key(26)
    M, N, K, G = 3, 9, 512, 128
    x = synth.activations(key, M, K)
    q, s = oracle.quant_act(synth.bf16_bits(x).numpy().view(np.uint16))
    packed = synth.random_bytes(synth.stream_key(key, 1), N * K // 4).numpy().reshape(N, K // 4)
    s_w = np.full((N, K // G), 0.0137, np.float32)
    acc_g, y_g = oracle.linear_grouped(q, s, packed, s_w, G)
    acc_t, y_t = oracle.linear(q, s, packed, np.float32(0.0137))
    assert np.array_equal(acc_g, acc_t)
    assert np.all(np.abs(y_g.astype(np.float64) - y_t) <= 2.0 ** -23 * np.abs(y_t.astype(np.float64)))


# ----------------------------------------------------------------- SwiGLU before down

def _silu_mul_exact_f32(g: float, u: float) -> float:
    """fp32 rounding of g u / (1 + e^-g), e^-g to 50 digits (decimal module)."""
    import decimal
    ctx = decimal.Context(prec=50)
    gd = decimal.Decimal(g)
    den = ctx.add(decimal.Decimal(1), ctx.exp(ctx.minus(gd)))
    val = ctx.divide(ctx.multiply(gd, decimal.Decimal(u)), den)
    return round_fraction_to_f32(Fraction(val))


def test_swiglu_quant_hand_case():
    """silu(0) = 0; silu(20) u rounds to 20 u (the factor 1 - 2e-9 is below half
    an fp32 unit); silu(1) 2 = 2 / (1 + 1/e) = 1.46211716..."""
    g = np.array([[0.0, 1.0, -1.0, 20.0]], np.float32)
    u = np.array([[3.0, 2.0, 2.0, 1.0]], np.float32)
    a, q, s = oracle.swiglu_quant(g, u)
    assert a[0, 0] == 0.0 and a[0, 3] == 20.0
    assert a[0, 1] == np.float32(2.0 / (1.0 + math.exp(-1.0)))
    assert a[0, 2] == np.float32(-2.0 / (1.0 + math.exp(1.0)))
    assert s[0] == 20.0
    # 127 a / 20 = 0, 9.284..., -3.415..., 127
    assert q.tolist() == [[0, 9, -3, 127]]


@pytest.mark.parametrize("K", [64, 300])
def test_swiglu_quant_exact(K):
    """a against the correctly rounded fp32 of g u / (1 + e^-g) (50-digit exp); codes
    against exact rational RNE of 127 a / max|a|."""
    key = synth.stream_key(27, K)
    M = 3
    g = (4.0 * synth.normal(key, M * K).float().numpy()).astype(np.float32).reshape(M, K)
    u = synth.normal(synth.stream_key(key, 1), M * K).float().numpy().astype(np.float32).reshape(M, K)
    a, q, s = oracle.swiglu_quant(g, u)
    for m in range(M):
        for k in range(K):
            assert a[m, k] == np.float32(_silu_mul_exact_f32(float(g[m, k]), float(u[m, k]))), (m, k)
        assert s[m] == np.abs(a[m]).max()
        for k in range(K):
            v = 127 * Fraction(float(a[m, k])) / Fraction(float(s[m]))
            fl = v.numerator // v.denominator
            rem = v - fl
            r = fl + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2) else 0)
            assert q[m, k] == r, (m, k)


def test_swiglu_quant_invariants():
    key = synth.stream_key(28)
    M, K = 4, 512
    g = (3.0 * synth.normal(key, M * K).float().numpy()).astype(np.float32).reshape(M, K)
    u = synth.normal(synth.stream_key(key, 1), M * K).float().numpy().astype(np.float32).reshape(M, K)
    a, q, s = oracle.swiglu_quant(g, u)
    # up -> -up negates a and the codes
    an, qn, sn = oracle.swiglu_quant(g, -u)
    assert np.array_equal(an, -a) and np.array_equal(qn, -q) and np.array_equal(sn, s)
    # up -> 2 up (exact) doubles a and s and keeps the codes
    a2, q2, s2 = oracle.swiglu_quant(g, 2 * u)
    assert np.array_equal(a2, 2 * a) and np.array_equal(q2, q) and np.array_equal(s2, 2 * s)
    # silu(g) > 0 for g > 0 and < 0 for g < 0, so with up = 1 the signs follow g
    a1, _, _ = oracle.swiglu_quant(g, np.ones_like(u))
    assert np.array_equal(np.sign(a1), np.sign(g))
    # silu(g) - silu(-g) = g: the two values of a differ by g to within rounding
    am, _, _ = oracle.swiglu_quant(-g, np.ones_like(u))
    assert np.all(np.abs((a1.astype(np.float64) - am) - g) <= 2.0 ** -23 * (np.abs(a1) + np.abs(am)))
    assert np.all(np.abs(q).max(axis=1) == 127)
    # a row with up = 0
    uz = u.copy()
    uz[1] = 0.0
    _, qz, sz = oracle.swiglu_quant(g, uz)
    assert not qz[1].any() and sz[1] == 0.0


# ----------------------------------------------------------------- fp32 rows

def _rne_fraction(v: Fraction) -> int:
    fl = v.numerator // v.denominator
    rem = v - fl
    return fl + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2) else 0)


def test_quant_act_f32_hand_case():
    q, s = oracle.quant_act_f32(np.array([[1.0, 2.0, 0.0, -1.0], [0.0, 0.0, 0.0, 0.0]], np.float32))
    assert q.tolist() == [[64, 127, 0, -64], [0, 0, 0, 0]] and s.tolist() == [2.0, 0.0]


def test_quant_act_f32_near_ties_exact():
    """x = fp32((2j + 1) / 254) with s = 1: 127 x lies within an fp32 rounding of
    j + 1/2, so only the exact quotient decides (binary32 arithmetic would not)."""
    j = np.arange(0, 127)
    x = np.concatenate([((2 * j + 1) / 254.0).astype(np.float32), [np.float32(1.0)]])
    x = np.stack([x, -x])
    q, s = oracle.quant_act_f32(x)
    assert s.tolist() == [1.0, 1.0]
    for m in range(2):
        for k in range(x.shape[1]):
            assert q[m, k] == _rne_fraction(127 * Fraction(float(x[m, k]))), (m, k)


def test_quant_act_f32_exact_random():
    key = synth.stream_key(29)
    M, K = 4, 700
    x = synth.normal(key, M * K).float().numpy().astype(np.float32).reshape(M, K)
    x[1] *= 1e-30
    x[2] *= 1e30
    q, s = oracle.quant_act_f32(x)
    for m in range(M):
        assert s[m] == np.abs(x[m]).max()
        for k in range(K):
            assert q[m, k] == _rne_fraction(127 * Fraction(float(x[m, k])) / Fraction(float(s[m]))), (m, k)


def test_swiglu_quant_codes_are_those_of_its_fp32_row():
    key = synth.stream_key(30)
    g = (3.0 * synth.normal(key, 3 * 640).float().numpy()).astype(np.float32).reshape(3, 640)
    u = synth.normal(synth.stream_key(key, 1), 3 * 640).float().numpy().astype(np.float32).reshape(3, 640)
    a, q, s = oracle.swiglu_quant(g, u)
    q2, s2 = oracle.quant_act_f32(a)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


# ----------------------------------------------------------------- binary (b1.0) weights

def test_pack_binary_hand_case():
    """w = [0.5, -0.25, 0, -0, 1, -2, 3, -4]: +1 for the first, third, fourth (both
    zeros), fifth and seventh -> bits 0, 2, 3, 4, 6 -> 0x5D; mean |w| = 10.75 / 8."""
    w = np.array([[0.5, -0.25, 0.0, -0.0, 1.0, -2.0, 3.0, -4.0]], np.float32)
    bits, s_w = oracle.pack_binary(w)
    assert bits.tolist() == [[0x5D]] and s_w == np.float32(10.75 / 8)


def _decode_binary(bits, K):
    b = np.unpackbits(bits.reshape(-1, 1), axis=1, bitorder="little").reshape(bits.shape[0], K)
    return (2 * b.astype(np.int64) - 1)


@pytest.mark.parametrize("M,N,K", [(1, 1, 8), (2, 3, 16), (3, 5, 256)])
def test_linear_binary_brute_force(M, N, K):
    key = synth.stream_key(31, M, N, K)
    q = synth.random_bytes(key, M * K).numpy().view(np.int8).reshape(M, K).copy()
    q[q == -128] = -127
    bits = synth.random_bytes(synth.stream_key(key, 1), N * K // 8).numpy().reshape(N, K // 8)
    s = np.linspace(0.5, 2.0, M).astype(np.float32)
    acc, y = oracle.linear_binary(q, s, bits, np.float32(0.03))
    t = _decode_binary(bits, K)
    for m in range(M):
        for n in range(N):
            a = sum(int(q[m, k]) * int(t[n, k]) for k in range(K))
            assert acc[m, n] == a
            exact = Fraction(a) * Fraction(float(s[m])) * Fraction(float(np.float32(0.03))) / 127
            assert assert_rescale_rounding(y[m, n], exact, abs(exact) * EPI_REL, (m, n))


def test_binary_of_weights_is_their_sign():
    """Packing then decoding gives sign(w) with zeros as +1; the linear of binary
    weights equals the ternary linear of the same +-1 values (codes 0 / 2)."""
    key = synth.stream_key(32)
    N, K = 6, 256
    w = synth.latent_weights(key, N, K, 0.02).numpy()
    w[0, :5] = 0.0
    bits, s_w = oracle.pack_binary(w)
    t = _decode_binary(bits, K)
    assert np.array_equal(t, np.where(w >= 0, 1, -1))
    codes = (t + 1).astype(np.uint8).reshape(N, K // 4, 4)
    packed = (codes[..., 0] | codes[..., 1] << 2 | codes[..., 2] << 4 | codes[..., 3] << 6).astype(np.uint8)
    x = synth.activations(synth.stream_key(key, 1), 3, K)
    q, s = oracle.quant_act(synth.bf16_bits(x).numpy().view(np.uint16))
    acc_b, y_b = oracle.linear_binary(q, s, bits, s_w)
    acc_t, y_t = oracle.linear(q, s, packed, s_w)
    assert np.array_equal(acc_b, acc_t) and np.array_equal(y_b, y_t)


# ----------------------------------------------------------------- sign / mask bitplanes

def test_bitplanes_hand_case():
    """Byte 0xA4 holds t = [-1, 0, +1, +1] (codes 0, 1, 2, 2); the rest of the 32
    weights are zero (byte 0x55): mask word 0b1101 = 0x0D, sign word 0b0001."""
    packed = np.array([[0xA4] + [0x55] * 7], np.uint8)
    planes = oracle.pack_bitplanes(packed, 32)
    assert planes.tolist() == [[[0x0D, 0, 0, 0, 0x01, 0, 0, 0]]]


def test_bitplanes_decode_and_linear_match_codes():
    key = synth.stream_key(33)
    N, K = 7, 640
    w = synth.latent_weights(key, N, K, 0.02).numpy()
    packed, s_w = oracle.pack(w)
    planes = oracle.pack_bitplanes(packed, K)
    # independent decode of the planes (numpy bit order) against the codes
    pb = np.unpackbits(planes.reshape(N, K // 32, 2, 4), axis=3, bitorder="little").reshape(N, K // 32, 2, 32)
    t = (pb[:, :, 0, :].astype(np.int64) * (1 - 2 * pb[:, :, 1, :].astype(np.int64))).reshape(N, K)
    assert np.array_equal(t, decode_unpackbits(packed, K))
    assert not np.any(pb[:, :, 1, :] & (1 - pb[:, :, 0, :]))      # no sign without the mask
    x = synth.activations(synth.stream_key(key, 1), 4, K)
    q, s = oracle.quant_act(synth.bf16_bits(x).numpy().view(np.uint16))
    acc_p, y_p = oracle.linear_bitplanes(q, s, planes, s_w)
    acc_t, y_t = oracle.linear(q, s, packed, s_w)
    assert np.array_equal(acc_p, acc_t) and np.array_equal(y_p, y_t)


def test_bitplanes_code3_becomes_plus_one():
    packed = np.array([[0xFF] * 8], np.uint8)                 # every code 3
    planes = oracle.pack_bitplanes(packed, 32)
    assert planes.tolist() == [[[0xFF, 0xFF, 0xFF, 0xFF, 0, 0, 0, 0]]]
