"""Pins for the oracle's decoders and its round-to-nearest-even helper.

The decoders are checked exhaustively against independent conversions
(numpy's binary16, torch's bfloat16 and OCP fp8 types); the rounding helper
against the binary16 worked example of the Tencent deterministic-inference
article (section "背景") stored in tests/golden, and against numpy/torch casts.
"""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp16_worked_example.txt")


def _read_golden():
    table, rounds, ulps = [], [], []
    with open(GOLDEN, encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            p = line.split()
            if p[0] == "round":
                rounds.append((float(p[1]), float(p[2])))
            elif p[0] == "ulp":
                ulps.append((float(p[1]), float(p[2])))
            else:
                table.append((float(p[0]), int(p[1], 2), int(p[2], 2)))
    return table, rounds, ulps


def _same(a, b):
    """Equal as fp64 values, NaN matched by class, zero matched by sign."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return np.all(both_nan | eq), np.flatnonzero(~(both_nan | eq))


# ---------------------------------------------------------------- decoders


def test_decode_f16_exhaustive():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    ok, bad = _same(oracle.decode("f16", bits), ref)
    assert ok, bad[:10]


def test_decode_bf16_exhaustive():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ok, bad = _same(oracle.decode("bf16", bits), ref)
    assert ok, bad[:10]


@pytest.mark.parametrize("fmt,tdt", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_decode_fp8_exhaustive(fmt, tdt):
    bits = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(bits.copy()).view(tdt).to(torch.float64).numpy()
    ok, bad = _same(oracle.decode(fmt, bits), ref)
    assert ok, bad[:10]


def test_decode_fp8_format_landmarks():
    # OCP FP8: e4m3fn has no infinities, max 448, NaN only at S.1111.111;
    # e5m2 is IEEE-like with max 57344 and infinities.
    d = oracle.decode("e4m3", np.array([0x7E, 0x7F, 0xFF, 0x01, 0x08], dtype=np.uint8))
    assert d[0] == 448.0 and np.isnan(d[1]) and np.isnan(d[2])
    assert d[3] == 2.0 ** -9 and d[4] == 2.0 ** -6
    d = oracle.decode("e5m2", np.array([0x7B, 0x7C, 0x7D, 0x01, 0x04], dtype=np.uint8))
    assert d[0] == 57344.0 and np.isinf(d[1]) and np.isnan(d[2])
    assert d[3] == 2.0 ** -16 and d[4] == 2.0 ** -14


def test_decode_f32_random():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    ok, bad = _same(oracle.decode("f32", bits), bits.view(np.float32).astype(np.float64))
    assert ok, bad[:10]


# ------------------------------------------------- the pages' worked example


def test_worked_example_encoding_table():
    table, _, _ = _read_golden()
    assert len(table) == 7
    for value, bexp, sig in table:
        want = (bexp << 10) | sig
        got = int(oracle.round_rne("f16", [value])[0])
        assert got == want, (value, hex(got), hex(want))
        assert oracle.decode("f16", np.array([want], dtype=np.uint16))[0] == value


def test_worked_example_2048_plus_1():
    _, rounds, ulps = _read_golden()
    for exact, rounded in rounds:
        b = oracle.round_rne("f16", [exact])
        assert oracle.decode("f16", b)[0] == rounded
    for at, ulp in ulps:
        b = int(oracle.round_rne("f16", [at])[0])
        nxt = oracle.decode("f16", np.array([b + 1], dtype=np.uint16))[0]
        assert nxt - at == ulp
    # 2049 has no binary16 encoding: both neighbours are 2 away from each other.
    assert 2049.0 not in oracle.decode("f16", np.arange(1 << 15, dtype=np.uint16))


def test_nonassociativity_fp16():
    # (2048 + 1) + 1 = 2048 but 2048 + (1 + 1) = 2050 when each sum is rounded to binary16.
    r = lambda x: oracle.decode("f16", oracle.round_rne("f16", [x]))[0]
    left = r(r(2048.0 + 1.0) + 1.0)
    right = r(2048.0 + r(1.0 + 1.0))
    assert left == 2048.0 and right == 2050.0


def test_nonassociativity_fp32():
    # Same argument one format up: ULP at 2^24 is 2 in binary32.
    r = lambda x: oracle.decode("f32", oracle.round_rne("f32", [x]))[0]
    t = 2.0 ** 24
    assert r(r(t + 1.0) + 1.0) == t
    assert r(t + r(1.0 + 1.0)) == t + 2.0


# ------------------------------------------------------- rounding vs casts


def _midpoints(fmt, np_bits_dtype, n, rng):
    """Exact halfway points between adjacent finite positive values of fmt."""
    top = {"f16": 0x7BFF, "bf16": 0x7F7F}[fmt]
    b = rng.integers(0, top, size=n).astype(np_bits_dtype)
    lo = oracle.decode(fmt, b)
    hi = oracle.decode(fmt, (b + 1).astype(np_bits_dtype))
    return (lo + hi) / 2.0  # exact in fp64 (p + 1 <= 53 bits)


def test_round_f16_vs_numpy():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(500_000) * 10.0 ** rng.integers(-9, 5, size=500_000),
        _midpoints("f16", np.uint16, 100_000, rng),
        -_midpoints("f16", np.uint16, 100_000, rng),
        np.array([0.0, -0.0, 65504.0, 65519.999, 65520.0, 1e6, 2.0 ** -24, 2.0 ** -25,
                  2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26]),
    ])
    got = oracle.round_rne("f16", x)
    want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want), np.flatnonzero(got != want)[:10]


def test_round_f32_vs_numpy():
    rng = np.random.default_rng(12)
    f32_bits = rng.integers(0, 0x7F7FFFFF, size=100_000).astype(np.uint32)
    lo = f32_bits.view(np.float32).astype(np.float64)
    hi = (f32_bits + 1).view(np.float32).astype(np.float64)
    x = np.concatenate([
        rng.standard_normal(500_000) * 10.0 ** rng.integers(-40, 38, size=500_000),
        (lo + hi) / 2.0, -(lo + hi) / 2.0,
        np.array([0.0, -0.0, 2.0 ** -149, 2.0 ** -150, 3.0 * 2.0 ** -151, 3.5e38]),
    ])
    got = oracle.round_rne("f32", x)
    want = x.astype(np.float32).view(np.uint32)
    assert np.array_equal(got, want), np.flatnonzero(got != want)[:10]


def test_round_bf16_vs_torch():
    # torch rounds fp32 -> bf16 with ties to even; feed values exact in fp32
    # so that its conversion is a single rounding.
    rng = np.random.default_rng(13)
    xs = (rng.standard_normal(500_000) * 10.0 ** rng.integers(-30, 30, size=500_000))
    xs = xs.astype(np.float32).astype(np.float64)
    mids = _midpoints("bf16", np.uint16, 100_000, rng)
    x = np.concatenate([xs, mids, -mids, np.array([0.0, -0.0, 1.0 + 2.0 ** -8,
                                                    1.0 + 3 * 2.0 ** -8])])
    got = oracle.round_rne("bf16", x)
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16)
    want = want.numpy().view(np.uint16)
    assert np.array_equal(got, want), np.flatnonzero(got != want)[:10]


def test_round_ties_to_even_f16():
    # 2051 lies halfway between 2050 (odd significand) and 2052 (even): goes up;
    # 2053 lies halfway between 2052 (even) and 2054: goes down.
    d = oracle.decode("f16", oracle.round_rne("f16", [2051.0, 2053.0, -2051.0]))
    assert list(d) == [2052.0, 2052.0, -2052.0]


def test_round_e4m3_vs_torch():
    # OCP e4m3fn: every finite value and every midpoint between neighbours
    # (ties to even), plus random values in range, against torch's cast of
    # fp32 inputs (all of them exact in fp32).
    allv = oracle.decode("e4m3", np.arange(256, dtype=np.uint8))
    fin = np.unique(allv[np.isfinite(allv)])
    mids = (fin[:-1] + fin[1:]) / 2.0
    rng = np.random.default_rng(14)
    xs = rng.uniform(-448.0, 448.0, 200_000).astype(np.float32).astype(np.float64)
    tiny = rng.uniform(-2.0 ** -6, 2.0 ** -6, 50_000).astype(np.float32).astype(np.float64)
    x = np.concatenate([fin, mids, xs, tiny, np.array([0.0, -0.0])])
    got = oracle.round_rne("e4m3", x)
    want = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(got, want.numpy()), np.flatnonzero(got != want.numpy())[:10]
    # 448 is the largest finite value; beyond it e4m3fn has only NaN
    assert oracle.round_rne("e4m3", [448.0, 464.0 - 1e-9, 1e6]).tolist()[:2] == [0x7E, 0x7E]
    assert oracle.round_rne("e4m3", [1e6])[0] & 0x7F == 0x7F
