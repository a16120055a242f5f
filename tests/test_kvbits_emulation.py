"""The host emulation of the RoPE kernel's float32 arithmetic (tests/kvbits.py)
against exact rational arithmetic: the fused multiply-add rounds the exact
a*b + c once to the nearest float32 (ties to even), including the cases where
a float64 intermediate sits exactly halfway between two float32 values."""
from fractions import Fraction

import numpy as np
import torch

from tests import kvbits


def _round_f32_exact(q: Fraction) -> np.float32:
    """Nearest float32 to the rational q, ties to the even significand."""
    r = np.float32(float(q))
    cands = {r, np.nextafter(r, np.float32(np.inf)), np.nextafter(r, np.float32(-np.inf))}
    best = None
    for c in cands:
        dist = abs(Fraction(float(c)) - q)
        key = (dist, int(np.float32(c).view(np.int32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def test_fmaf_halfway_float64_sum():
    # 24929 * 673 / 2^24 = 1 + 2^-24 exactly: halfway between 1 and 1 + 2^-23.
    a = np.float32(24929.0)
    b = np.float32(673.0 / 2 ** 24)
    assert Fraction(float(a)) * Fraction(float(b)) == 1 + Fraction(1, 2 ** 24)
    tiny = np.float32(2.0 ** -80)
    assert kvbits.fmaf(a, b, tiny) == np.float32(1 + 2 ** -23)      # just above halfway: up
    assert kvbits.fmaf(a, b, -tiny) == np.float32(1.0)              # just below: down
    assert kvbits.fmaf(a, b, np.float32(0.0)) == np.float32(1.0)    # exact tie: even
    # a plain float64 sum cast to float32 gets the first case wrong
    assert np.float32(float(a) * float(b) + float(tiny)) == np.float32(1.0)


def test_fmaf_random_against_rationals():
    rng = np.random.default_rng(5)
    n = 3000
    a = (rng.standard_normal(n) * np.exp2(rng.integers(-8, 8, n))).astype(np.float32)
    b = rng.uniform(-1, 1, n).astype(np.float32)
    c = (rng.standard_normal(n) * np.exp2(rng.integers(-30, 4, n))).astype(np.float32)
    got = kvbits.fmaf(a, b, c)
    for i in range(n):
        q = Fraction(float(a[i])) * Fraction(float(b[i])) + Fraction(float(c[i]))
        assert got[i] == _round_f32_exact(q), (i, a[i], b[i], c[i])


def test_rotation_and_bf16_bits():
    rng = np.random.default_rng(6)
    x0 = torch.randn(500).bfloat16().float().numpy()
    x1 = torch.randn(500).bfloat16().float().numpy()
    ang = rng.uniform(0, 100, 500)
    c, s = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    y0, y1 = kvbits.rope_fp32(x0, x1, c, s)
    for i in range(500):
        q0 = Fraction(float(x0[i])) * Fraction(float(c[i])) - Fraction(float(_round_f32_exact(
            Fraction(float(x1[i])) * Fraction(float(s[i])))))
        q1 = Fraction(float(x1[i])) * Fraction(float(c[i])) + Fraction(float(_round_f32_exact(
            Fraction(float(x0[i])) * Fraction(float(s[i])))))
        assert y0[i] == _round_f32_exact(q0) and y1[i] == _round_f32_exact(q1)
    # bf16 bits: torch's conversion rounds to nearest even
    bits = kvbits.to_bits(np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8], np.float32), "bf16")
    assert bits.tolist() == [0x3F80, 0x3F82]
