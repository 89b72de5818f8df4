"""Pins of the oracle's numeric primitives against closed forms, textbook or
library routines, invariants and brute force (CPU only)."""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(x):
    return np.float32(x)


# ---------------------------------------------------------------- bf16 ----

def test_bf16_rounding_matches_torch(orc):
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    # ties: low 16 bits exactly 0x8000
    ties = (rng.integers(0, 2**16, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.f32_to_bf16_bits(x[:3000])
    assert np.array_equal(got, ref[:3000])
    assert np.array_equal(orc.round_bf16(x), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_bf16_rounding_cases(orc):
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: round to even (1.0)
    assert orc.f32_to_bf16_bits(np.array([1 + 2.0**-8], np.float32))[0] == 0x3F80
    # 1 + 3*2^-8 ties between 1+2^-7 (odd mantissa) and 1+2^-6: round up to even
    assert orc.f32_to_bf16_bits(np.array([1 + 3 * 2.0**-8], np.float32))[0] == 0x3F82
    nan = orc.f32_to_bf16_bits(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0
    assert orc.f32_to_bf16_bits(np.array([np.float32(3.4e38)], np.float32))[0] == 0x7F80  # -> inf


# ---------------------------------------------------------------- RoPE ----

def test_rope_table_angles(orc):
    T, D, theta = 64, 16, 10000.0
    cos, sin = orc.rope_table(T, D, theta)
    t = np.arange(T, dtype=np.float64)[:, None]
    inv = np.array([theta ** (-2.0 * j / D) for j in range(D // 2)])
    a = t * inv[None, :]
    # fp64 library cosine rounded to fp32: at most one fp32 rounding apart
    assert np.all(np.abs(cos - np.cos(a).astype(np.float32)) <= np.spacing(np.abs(cos)) + 1e-30)
    assert np.all(np.abs(sin - np.sin(a).astype(np.float32)) <= np.spacing(np.abs(sin)) + 1e-30)
    assert np.all(cos[0] == 1.0) and np.all(sin[0] == 0.0)


@pytest.mark.parametrize("style", [0, 1])
def test_rope_forward_is_rotation(orc, style):
    """Forward RoPE equals the complex rotation (x_a + i x_b) e^{i t w_j}."""
    rng = np.random.default_rng(1)
    D, T, theta = 64, 300, 5e5
    cos, sin = orc.rope_table(T, D, theta)
    for t in (0, 1, 7, 299):
        x = rng.standard_normal(D).astype(np.float32)
        y = orc.rope_forward(x, cos[t], sin[t], style)
        if style == 0:
            a, b = np.arange(D // 2), np.arange(D // 2) + D // 2
        else:
            a, b = np.arange(0, D, 2), np.arange(1, D, 2)
        z = (x[a].astype(np.float64) + 1j * x[b]) * np.exp(1j * t * theta ** (-2.0 * np.arange(D // 2) / D))
        tol = 4 * np.spacing(np.maximum(np.abs(x[a]), np.abs(x[b])).astype(np.float32))
        assert np.all(np.abs(y[a] - z.real) <= tol)
        assert np.all(np.abs(y[b] - z.imag) <= tol)


@pytest.mark.parametrize("style", [0, 1])
def test_rope_inverse_undoes_forward(orc, style):
    rng = np.random.default_rng(2)
    D, T, theta = 128, 4096, 5e5
    cos, sin = orc.rope_table(T, D, theta)
    for t in rng.integers(0, T, 40):
        x = rng.standard_normal(D).astype(np.float32) * 3
        y = orc.rope_forward(x, cos[t], sin[t], style)
        xr = orc.rope_inverse(y, cos[t], sin[t], style)
        if style == 0:
            mag = np.maximum(np.abs(x[: D // 2]), np.abs(x[D // 2:]))
            mag = np.concatenate([mag, mag])
        else:
            mag = np.repeat(np.maximum(np.abs(x[0::2]), np.abs(x[1::2])), 2)
        assert np.all(np.abs(xr - x) <= 4 * np.spacing(mag.astype(np.float32)))
    # position 0: cos = 1 and sin = 0, the inverse is bit-exact
    x = rng.standard_normal(D).astype(np.float32)
    assert np.array_equal(orc.rope_inverse(x, cos[0], sin[0], style), x)


def test_rope_unit_vector(orc):
    D, theta = 16, 100.0
    cos, sin = orc.rope_table(3, D, theta)
    for j in range(D // 2):
        e = np.zeros(D, np.float32)
        e[j] = 1
        y = orc.rope_forward(e, cos[1], sin[1], 0)
        w = theta ** (-2.0 * j / D)
        assert y[j] == np.float32(math.cos(w)) and y[j + D // 2] == np.float32(math.sin(w))


# ---------------------------------------------------------- projection ----

def _bf16_values(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).float().numpy()


def test_projection_is_correctly_rounded_exact_sum(orc):
    """bf16 operands: c_i = fp32(exact sum), checked with rational arithmetic."""
    rng = np.random.default_rng(3)
    D = 16
    for _ in range(20):
        x = _bf16_values(rng, D, 5.0)
        B = _bf16_values(rng, (D, D), 0.3)
        c = orc.project(x, B)
        for i in range(D):
            exact = sum(Fraction(float(x[j])) * Fraction(float(B[j, i])) for j in range(D))
            assert c[i] == np.float32(float(exact))  # float(Fraction) rounds correctly


def test_projection_special_bases(orc):
    rng = np.random.default_rng(4)
    D = 64
    x = rng.standard_normal(D).astype(np.float32)
    assert np.array_equal(orc.project(x, np.eye(D, dtype=np.float32)), x)
    perm = rng.permutation(D)
    P = np.eye(D, dtype=np.float32)[:, perm]  # column i = e_{perm[i]}
    assert np.array_equal(orc.project(x, P), x[perm])
    assert np.array_equal(orc.unproject(x[perm], P), x)


def test_transform_round_trip_sanity_row(orc):
    """Codec-Gauge 'Evaluation Design' sanity rows: G^-1 G round trip with
    NRMSE below 5.1e-8 (fp32 operands, random orthogonal gauge)."""
    rng = np.random.default_rng(5)
    D, N = 128, 400
    Q = scipy.linalg.qr(rng.standard_normal((D, D)))[0].astype(np.float32)
    x = rng.standard_normal((N, D)).astype(np.float32)
    c = np.stack([orc.project(r, Q) for r in x])
    xr = np.stack([orc.unproject(r, Q) for r in c])
    nrmse = math.sqrt(float(((xr.astype(np.float64) - x) ** 2).sum() / (x.astype(np.float64) ** 2).sum()))
    assert nrmse < 5.1e-8, nrmse
    # Parseval: an orthogonal basis keeps the norm
    assert np.allclose(np.linalg.norm(c, axis=1), np.linalg.norm(x, axis=1), rtol=1e-5)


# ----------------------------------------------------------------- WHT ----

def test_wht_h2_closed_form(orc):
    y = orc.wht(np.array([3.0, 1.0], np.float32))
    assert y[0] == np.float32(4 / math.sqrt(2)) and y[1] == np.float32(2 / math.sqrt(2))


@pytest.mark.parametrize("D", [4, 16, 64, 128])
def test_wht_matches_sylvester_hadamard(orc, D):
    """scipy.linalg.hadamard builds the Sylvester-order matrix."""
    rng = np.random.default_rng(6)
    H = scipy.linalg.hadamard(D).astype(np.float64)
    for _ in range(10):
        x = _bf16_values(rng, D, 2.0)
        ref = (H @ x.astype(np.float64) / math.sqrt(D)).astype(np.float32)
        assert np.array_equal(orc.wht(x), ref)
    # H H^T = D I, recovered from the transform of unit vectors
    Hr = np.stack([orc.wht(np.eye(D, dtype=np.float32)[j]) for j in range(D)], axis=1) * math.sqrt(D)
    assert np.allclose(Hr @ Hr.T, D * np.eye(D), atol=1e-4)


def test_wht_is_involution(orc):
    rng = np.random.default_rng(7)
    x = rng.standard_normal(128).astype(np.float32)
    xr = orc.wht(orc.wht(x))
    assert np.all(np.abs(xr - x) <= 4 * np.spacing(np.float32(np.abs(x).max())))


def test_rms(orc):
    """Closed forms of the root mean square over the D entries of a row: a
    constant row gives its magnitude, a single spike of a in D entries gives
    |a| / sqrt(D), an alternating row +-a gives |a|, (3, 4) gives 5/sqrt(2),
    and scaling by a power of two scales the result exactly."""
    assert orc.rms(np.full(128, 3.0, np.float32)) == np.float32(3.0)
    assert orc.rms(np.full(64, -0.75, np.float32)) == np.float32(0.75)
    spike = np.zeros(64, np.float32)
    spike[17] = -24.0
    assert orc.rms(spike) == np.float32(3.0)  # 24 / sqrt(64)
    alt = np.array([5.5, -5.5] * 64, np.float32)
    assert orc.rms(alt) == np.float32(5.5)
    assert orc.rms(np.array([3.0, 4.0], np.float32)) == np.float32(5.0 / math.sqrt(2.0))
    assert orc.rms(np.zeros(128, np.float32)) == 0.0
    rng = np.random.default_rng(8)
    x = _bf16_values(rng, 128, 3.0)
    assert orc.rms(x * np.float32(8.0)) == np.float32(8.0) * orc.rms(x)


# --------------------------------------------------------------- stats ----

def test_stats_against_numpy(orc):
    rng = np.random.default_rng(9)
    c = (rng.standard_normal((1000, 32)) * 3 + 1.5).astype(np.float32)
    mu, var, mn, mx = orc.stats(c)
    c64 = c.astype(np.float64)
    assert np.allclose(mu, c64.mean(0), rtol=1e-6, atol=0)
    assert np.allclose(var, c64.var(0), rtol=1e-6, atol=0)
    assert np.array_equal(mn, c.min(0)) and np.array_equal(mx, c.max(0))
    const = np.full((50, 4), 2.5, np.float32)
    mu, var, mn, mx = orc.stats(const)
    assert np.all(var == 0) and np.all(mu == 2.5) and np.all(mn == mx)


# ---------------------------------------------------------- allocation ----

def test_budget(orc):
    assert orc.budget(1.6, 128) == 204
    assert orc.budget(2.0, 128) == 256
    assert orc.budget(4.0, 64) == 256
    assert orc.budget(1.0, 128) == 128


def test_greedy_hand_example(orc):
    # var 16, 4, 1; budget 3: 16 -> b0=1 (now 4), tie 4 vs 4 -> lowest index b0=2 (now 1),
    # then 4 (comp 1) -> [2, 1, 0]
    assert list(orc.alloc_greedy(np.array([16, 4, 1], np.float32), 3, 8)) == [2, 1, 0]
    assert list(orc.alloc_greedy(np.array([1, 1, 1], np.float32), 1, 8)) == [1, 0, 0]
    assert list(orc.alloc_greedy(np.array([0, 5, 0], np.float32), 20, 8)) == [0, 8, 0]
    assert list(orc.alloc_greedy(np.array([1, 1], np.float32), 100, 3)) == [3, 3]


def test_greedy_equals_brute_force(orc):
    rng = np.random.default_rng(10)
    for trial in range(60):
        D = int(rng.integers(1, 5))
        B = int(rng.integers(0, 9))
        mb = int(rng.integers(1, 5))
        var = np.exp(rng.uniform(-6, 6, D)).astype(np.float32)
        if trial % 5 == 0:
            var[rng.integers(0, D)] = 0
        g = orc.alloc_greedy(var, B, mb)
        best = min(orc.distortion(var, np.array(b, np.uint8))
                   for b in itertools.product(range(mb + 1), repeat=D) if sum(b) <= B)
        assert orc.distortion(var, g) == pytest.approx(best, rel=1e-12, abs=0)
        assert int(g.sum()) <= B


def test_greedy_equals_dp(orc):
    """The explainer's 'dynamic programming in the reference path' and the
    'greedier' path reach the same modelled distortion (convex separable cost)."""
    rng = np.random.default_rng(11)
    for _ in range(30):
        D = int(rng.integers(2, 33))
        B = int(rng.integers(0, 3 * D))
        var = np.exp(rng.uniform(-10, 10, D)).astype(np.float32)
        g = orc.alloc_greedy(var, B, 8)
        d, _ = orc.alloc_dp(var, B, 8)
        assert orc.distortion(var, g) == pytest.approx(d, rel=1e-12)


# ------------------------------------------------------- quantisation ----

def test_quantizer_half_step_bound(orc):
    rng = np.random.default_rng(12)
    c = (rng.standard_normal((3000, 16)) * np.exp(rng.uniform(-3, 3, 16))).astype(np.float32)
    mu, var, mn, mx = orc.stats(c)
    bits = np.array([0, 1, 2, 3, 4, 5, 6, 7, 8, 8, 2, 3, 1, 0, 4, 5], np.uint8)
    zero, scale, rcp = orc.side_info(bits, mu, mn, mx)
    q, v = orc.quantize(c, bits, zero, rcp)
    assert np.all(q <= ((1 << bits.astype(np.int64)) - 1))
    # decode: fma(q, scale, zero); fp64 evaluation differs from it by at most one rounding
    chat = (q.astype(np.float64) * scale.astype(np.float64) + zero.astype(np.float64)).astype(np.float32)
    for i in range(16):
        if bits[i] == 0:
            assert np.all(chat[:, i] == mu[i])
            continue
        err = np.abs(chat[:, i].astype(np.float64) - c[:, i])
        assert err.max() <= scale[i] / 2 + 8 * np.spacing(np.float32(np.abs(c[:, i]).max())), i


def test_quantizer_round_half_even_and_grid(orc):
    # zero = 0, scale = 1 (rcp = 1): v is exact, ties go to even
    c = np.array([[0.5], [1.5], [2.5], [3.0], [-0.2], [9.0]], np.float32)
    q, v = orc.quantize(c, np.array([3], np.uint8), np.array([0], np.float32), np.array([1], np.float32))
    assert list(q[:, 0]) == [0, 2, 2, 3, 0, 7]
    # lattice data m + k s with a power-of-two step: lossless
    rng = np.random.default_rng(13)
    k = rng.integers(0, 16, (200, 4))
    k[0], k[1] = 0, 15  # the range is exactly [m, m + 15 s]
    c = (1.25 + k * 0.125).astype(np.float32)
    mu, var, mn, mx = orc.stats(c)
    bits = np.full(4, 4, np.uint8)
    zero, scale, rcp = orc.side_info(bits, mu, mn, mx)
    assert np.all(scale == 0.125)
    q, _ = orc.quantize(c, bits, zero, rcp)
    assert np.array_equal(q, k.astype(np.uint8))


def test_symmetric_quantizer(orc):
    c = np.array([[-7.0, 7.0, 0.0, 3.5, -100.0, 2.49]], np.float32)
    q, _ = orc.quantize_sym(c, 4, 1.0)
    assert list(q[0]) == [1, 15, 8, 12, 1, 10]  # 3.5 -> 4 (even), clamp -7, offset 8


# ------------------------------------------------------------- packing ----

def test_pack_golden_example(orc):
    g = json.load(open(os.path.join(GOLDEN, "pack_example.json")))
    q = np.array(g["codes_token_major"], np.uint8)
    bits = np.array(g["bits"], np.uint8)
    out = orc.pack(q, bits)
    assert list(out) == g["packed"]
    back = orc.unpack(out, q.shape[0], bits)
    assert np.array_equal(back[:, [0, 2]], q[:, [0, 2]]) and np.all(back[:, 1] == 0)


def test_pack_round_trip(orc):
    rng = np.random.default_rng(14)
    for n in [0, 1, 2, 3, 31, 32, 33, 100, 257, 2000]:
        bits = rng.integers(0, 9, 12).astype(np.uint8)
        q = (rng.integers(0, 256, (n, 12)) & ((1 << bits.astype(np.int64)) - 1)).astype(np.uint8)
        data = orc.pack(q, bits)
        assert data.size == sum(4 * ((n * int(b) + 31) // 32) for b in bits if b)
        assert np.array_equal(orc.unpack(data, n, bits), q)


def test_binding_keeps_strided_arguments_alive(orc):
    """Strided views are copied to contiguous temporaries on their way into
    the C routines; each temporary must outlive the call (three of them at
    once here, whose memory would otherwise be reused by the next)."""
    rng = np.random.default_rng(3)
    st = rng.normal(size=(64, 4)).astype(np.float32)
    st[:, 3] = st[:, 2] + np.abs(st[:, 3]) + 1
    bits = np.full(64, 3, np.uint8)
    z, s, _ = orc.side_info(bits, st[:, 0], st[:, 2], st[:, 3])
    assert np.array_equal(z, st[:, 2])
    assert np.array_equal(s, ((st[:, 3].astype(np.float64) - st[:, 2]) / 7).astype(np.float32))
