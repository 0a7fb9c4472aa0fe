"""Pins of the oracle's packed projection (msa_oracle_project) and of its binary64 -> bf16 rounding,
against references that share nothing with it: exact rational arithmetic (fractions.Fraction) with a
nearest-code search over every bf16 value decoded from the format definition, numpy's binary64
matrix product on inputs where it is exact, and closed forms (one-hot weight rows pick input
columns; doubling the weights doubles every output)."""
import ctypes
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle


def bf16_exact(code: int) -> Fraction:
    """The exact value of a finite bf16 code: the upper half of a binary32."""
    return Fraction(struct.unpack("<f", struct.pack("<I", code << 16))[0])


_POS = None


def positive_grid():
    """All finite non-negative bf16 codes in ascending value order, with their exact values."""
    global _POS
    if _POS is None:
        codes = [c for c in range(0x0000, 0x7F80)]        # +0 .. largest finite
        _POS = (codes, [bf16_exact(c) for c in codes])
    return _POS


def nearest_bf16(v: Fraction) -> int:
    """Round an exact rational to bf16: nearest value, ties to the even code, overflow to
    infinity at or beyond the midpoint between the largest finite value and 2^128."""
    import bisect
    codes, vals = positive_grid()
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    top = vals[-1]
    if a >= top + (Fraction(2) ** 128 - top) / 2:
        return sign | 0x7F80
    i = bisect.bisect_left(vals, a)
    if i == len(vals):                                    # above the largest finite, below the midpoint
        return sign | codes[-1]
    if vals[i] == a:
        return sign | codes[i]
    lo, hi = i - 1, i
    dlo, dhi = a - vals[lo], vals[hi] - a
    if dlo < dhi or (dlo == dhi and codes[lo] % 2 == 0):
        return sign | codes[lo]
    return sign | codes[hi]


def test_bf16_of_f64_against_exact_rounding():
    rng = np.random.default_rng(11)
    vals = list(rng.standard_normal(300) * np.exp2(rng.integers(-140, 127, 300)))
    # exact ties and near-ties that a binary32 intermediate would round differently
    for e in (-130, -126, -20, 0, 5, 120):
        for m in (1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -40, 1 + 2 ** -8 - 2 ** -40,
                  1 + 2 ** -7 + 2 ** -8, 1.5 + 2 ** -9 + 2 ** -45):
            vals += [m * 2.0 ** e, -m * 2.0 ** e]
    top = float(bf16_exact(0x7F7F))
    vals += [0.0, -0.0, top, -top, 2.0 ** 128 * (1 - 2 ** -9), 2.0 ** 128 * (1 - 2 ** -9) * (1 - 2 ** -30),
             2.0 ** -133, 2.0 ** -134, 2.0 ** -134 * 1.0000001, 3 * 2.0 ** -135, 1e-300]
    for v in vals:
        got = oracle.bf16_of_f64(v)
        want = nearest_bf16(Fraction(v))
        if v == 0.0 or (want & 0x7FFF) == 0:
            want = (0x8000 if np.signbit(v) else 0) | (want & 0x7FFF)
        assert got == want, f"{v!r}: got 0x{got:04x}, want 0x{want:04x}"


def test_bf16_of_f64_agrees_with_binary32_encoder_on_binary32_values():
    """On values a binary32 holds exactly, rounding from binary64 or from binary32 is the same
    single rounding (the binary32 encoder is pinned by the exhaustive sweep)."""
    rng = np.random.default_rng(12)
    u = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    enc = oracle.encode_bf16(f)
    for v, e in zip(f[:4000], enc[:4000]):
        assert oracle.bf16_of_f64(float(v)) == int(e), float(v)


def _bits(a):
    return oracle.encode_bf16(np.asarray(a, np.float32))


def test_one_hot_weights_pick_input_columns():
    rng = np.random.default_rng(13)
    T, K, N = 9, 64, 40
    h = _bits(rng.standard_normal((T, K)).astype(np.float32)).reshape(T, K)
    pick = rng.integers(0, K, N)
    w = np.zeros((N, K), np.float32)
    w[np.arange(N), pick] = 1.0
    x = oracle.project(h, _bits(w).reshape(N, K))
    np.testing.assert_array_equal(x, h[:, pick])
    # a one-hot of weight -2 picks, negates and doubles (exactly)
    w2 = np.zeros((N, K), np.float32)
    w2[np.arange(N), pick] = -2.0
    x2 = oracle.project(h, _bits(w2).reshape(N, K))
    hv = (h.astype(np.uint32) << 16).view(np.float32)
    np.testing.assert_array_equal(x2, _bits(-2.0 * hv[:, pick]).reshape(T, N))


def test_dyadic_inputs_match_numpy_product_exactly():
    """Inputs on a coarse dyadic grid: every binary64 partial sum is exact, so numpy's product
    (any summation order) is the exact sum; rounded by the rational reference it must equal the
    oracle bit for bit."""
    rng = np.random.default_rng(14)
    T, K, N = 17, 96, 23
    hv = rng.integers(-64, 65, (T, K)) / 16.0
    wv = rng.integers(-32, 33, (N, K)) / 64.0
    x, sm, _ = oracle.project(_bits(hv).reshape(T, K), _bits(wv).reshape(N, K), want_sums=True)
    ref = hv @ wv.T
    np.testing.assert_array_equal(sm, ref)
    want = np.array([nearest_bf16(Fraction(v)) for v in ref.reshape(-1)], np.uint16).reshape(T, N)
    np.testing.assert_array_equal(x, want)


def test_random_normal_inputs_match_exact_rational_sum():
    rng = np.random.default_rng(15)
    T, K, N = 4, 24, 6
    h = _bits(rng.standard_normal((T, K)).astype(np.float32)).reshape(T, K)
    w = _bits((rng.standard_normal((N, K)) * 0.05).astype(np.float32)).reshape(N, K)
    x, sm, ab = oracle.project(h, w, want_sums=True)
    hv = [[bf16_exact(int(c)) for c in row] for row in h]
    wv = [[bf16_exact(int(c)) for c in row] for row in w]
    for t in range(T):
        for c in range(N):
            exact = sum(a * b for a, b in zip(hv[t], wv[c]))
            assert Fraction(sm[t, c]) == exact
            assert Fraction(ab[t, c]) == sum(abs(a * b) for a, b in zip(hv[t], wv[c]))
            assert x[t, c] == nearest_bf16(exact), (t, c)


def test_doubling_weights_doubles_outputs_and_rows_are_independent():
    rng = np.random.default_rng(16)
    T, K, N = 12, 128, 30
    h = _bits(rng.standard_normal((T, K)).astype(np.float32)).reshape(T, K)
    wf = (rng.standard_normal((N, K)) * 0.1).astype(np.float32)
    w = _bits(wf).reshape(N, K)
    w2 = _bits(2.0 * ((w.astype(np.uint32) << 16).view(np.float32))).reshape(N, K)
    x1, x2 = oracle.project(h, w), oracle.project(h, w2)
    v1 = (x1.astype(np.uint32) << 16).view(np.float32)
    v2 = (x2.astype(np.uint32) << 16).view(np.float32)
    np.testing.assert_array_equal(v2, 2.0 * v1)
    # a row's result does not depend on the other rows (no index mix-up between t and c)
    np.testing.assert_array_equal(oracle.project(h[5:6], w), x1[5:6])
    np.testing.assert_array_equal(oracle.project(h, w[7:8]), x1[:, 7:8])


def test_strided_views():
    """Row strides larger than the row length read and write only the view."""
    rng = np.random.default_rng(17)
    T, K, N = 5, 32, 7
    h = _bits(rng.standard_normal((T, K + 8)).astype(np.float32)).reshape(T, K + 8)
    w = _bits(rng.standard_normal((N, K + 16)).astype(np.float32)).reshape(N, K + 16)
    x = np.full((T, N + 3), 0x1234, np.uint16)
    L = oracle.lib()
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    assert L.msa_oracle_project(p(h), K + 8, T, K, p(w), K + 16, N, p(x), N + 3, None, None, 1) == 0
    np.testing.assert_array_equal(x[:, :N], oracle.project(h[:, :K], w[:, :K]))
    assert np.all(x[:, N:] == 0x1234)
    assert L.msa_oracle_project(p(h), K - 1, T, K, p(w), K + 16, N, p(x), N + 3, None, None, 1) != 0
