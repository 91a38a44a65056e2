"""The E4M3 quantiser's quotient without a division per value, checked as arithmetic on the CPU.

The device quantiser (shared by the quantising cache write and the appending decode kernels) forms x / scale as
q = RN(x * inv) with inv = RN(1 / scale), the exact residual r = x - q * scale (one fma), and RN(q + r * inv) (a
second fma), keeping q when r is zero or q is not finite, for |scale| in [2^-32, 2^32]. This test replays that
sequence in float32 with an exactly emulated fma and compares it with IEEE float32 division: equal for every
quotient that decides an E4M3 code (|x / scale| in [2^-11, 512)); smaller quotients only have to keep the sign of
the division's (they all give a zero code). The GPU tests compare the device codes with the oracle's on every
bf16 value; this one pins the arithmetic itself over far more scales.
"""
import numpy as np
import pytest


def fma32(a, b, c):
    """float32 a * b + c rounded once: the product is exact in float64 (24 x 24 bits), the sum is rounded to odd
    in float64 (53 >= 24 + 2 bits), so one rounding to float32 is the correctly rounded fma."""
    p = a.astype(np.float64) * b.astype(np.float64)
    c64 = c.astype(np.float64)
    s = p + c64
    bb = s - p
    err = (p - (s - bb)) + (c64 - bb)  # two-sum error of the float64 addition
    fix = (err != 0) & np.isfinite(s) & ((s.view(np.uint64) & 1) == 0)
    s = np.where(fix, np.nextafter(s, np.where(err > 0, np.inf, -np.inf)), s)
    return s.astype(np.float32)


def quotient(x, scale):
    s = np.float32(scale)
    inv = np.float32(1.0) / s
    q = x * inv
    r = fma32(-q, np.full_like(x, s), x)
    y = fma32(r, np.full_like(x, inv), q)
    return np.where((r == 0) | ~np.isfinite(q), q, y)


def check(x, scale):
    with np.errstate(over="ignore", invalid="ignore"):
        ref = x / np.float32(scale)
        got = quotient(x, scale)
    decides = (np.abs(ref) >= 2.0 ** -11) & (np.abs(ref) < 512)
    same = (ref.view(np.uint32) == got.view(np.uint32)) | (np.isnan(ref) & np.isnan(got))
    assert same[decides].all(), (scale, x[decides & ~same][:4])
    small = np.abs(ref) < 2.0 ** -11
    assert (np.signbit(ref[small]) == np.signbit(got[small])).all()
    assert (np.abs(got[small]) < 2.0 ** -10).all()


SCALES = np.concatenate([[1 / 64, 0.0125, 1 / 3, 0.3, 3.0, 7.0, -0.7, 2.0 ** -32, 1.999 * 2.0 ** 31],
                         np.random.default_rng(11).uniform(0.5, 1.0, 15) * 2.0 ** np.arange(-28, 30, 4)])


@pytest.mark.parametrize("scale", SCALES.astype(np.float32).tolist())
def test_every_bf16_value(scale):
    x = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
    check(x[np.isfinite(x)], scale)


def test_random_float32_values():
    rng = np.random.default_rng(12)
    for _ in range(8):
        scale = np.float32(rng.uniform(0.5, 1.0) * 2.0 ** int(rng.integers(-30, 30)))
        x = rng.integers(0, 2 ** 32, 200_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
        check(x[np.isfinite(x)], scale)
