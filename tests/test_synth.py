"""The seeded generator: known-answer hash, determinism, distributions, bf16 rounding."""
import math
from fractions import Fraction

import numpy as np
import pytest

import synth


def test_splitmix64_known_answer():
    # SplitMix64 (Steele, Lea, Flood 2014) started from state 0: published first outputs.
    got = synth.uniform_bytes(0, 24).view(np.uint64).tolist()
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_pure_function_of_indices():
    a = synth.experts(1000, 0, 3, 2, 4, 512, 128)
    b = synth.experts(1000, 0, 4, 1, 4, 512, 128)
    np.testing.assert_array_equal(a.gate[1], b.gate[0])
    np.testing.assert_array_equal(a.scales[1], b.scales[0])
    c = synth.experts(1001, 0, 4, 1, 4, 512, 128)
    assert not np.array_equal(b.gate, c.gate)
    d = synth.experts(1000, 1, 4, 1, 4, 512, 128)
    assert not np.array_equal(b.biases, d.biases)


def _bf16_rne_exact(v):
    """Nearest bf16 to v (ties to even), by exact rational search."""
    fv = Fraction(v)
    if fv == 0:
        return 0
    sign = 0x8000 if fv < 0 else 0
    a = abs(fv)
    e = math.floor(math.log2(a)) if a > 0 else 0
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (max(e, -126) - 7)
    n = a / q
    lo = math.floor(n)
    r = n - lo
    k = lo + (1 if (r > Fraction(1, 2) or (r == Fraction(1, 2) and lo % 2 == 1)) else 0)
    val = k * q
    f = np.array([float(val)], np.float32).view(np.uint32)[0]
    return sign | int(f >> 16)


def test_bf16_rounding_single_step():
    rng = np.random.default_rng(0)
    vals = list(rng.normal(0, 0.02, 2000)) + [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -40,
                                                -(1.0 + 2 ** -8), 2.0 ** -130, 1.5 * 2.0 ** -133]
    for v in vals:
        assert synth.bf16_from_double(float(v)) == _bf16_rne_exact(float(v)), v


def test_value_distributions():
    c = synth.experts(1000, 0, 0, 2, 4, 4096, 1024)
    nib = np.concatenate([c.gate.reshape(-1) & 15, c.gate.reshape(-1) >> 4])
    counts = np.bincount(nib, minlength=16) / nib.size
    assert np.all(np.abs(counts - 1 / 16) < 2e-3)
    f = lambda u16: (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    s, b = f(c.scales.reshape(-1)), f(c.biases.reshape(-1))
    assert np.all(s >= 0)
    assert abs(s.mean() - 0.02 * math.sqrt(2 / math.pi)) < 2e-4
    assert abs(b.std() - 0.01) < 1e-4 and abs(b.mean()) < 1e-4
    c2 = synth.experts(1002, 0, 0, 1, 2, 4096, 1024)
    crumbs = np.concatenate([(c2.up.reshape(-1) >> (2 * t)) & 3 for t in range(4)])
    assert np.all(np.abs(np.bincount(crumbs, minlength=4) / crumbs.size - 0.25) < 2e-3)


def test_router_and_token_distributions():
    W = synth.router(1001, 0, 512, 4096)
    assert abs(W.std() - 1 / 64) < 2e-4
    x = synth.tokens(1001, 0, 8, 4096)
    assert abs(x.std() - 1) < 0.02 and abs(x.mean()) < 0.02
    np.testing.assert_array_equal(synth.tokens(1001, 0, 8, 4096), x)
    assert not np.array_equal(synth.tokens(1001, 1, 8, 4096), x)


def test_zipf_prior():
    b = synth.zipf_bias(512, 1.1)
    assert b[0] == 0.0
    assert b[511] == np.float32(-1.1 * math.log(512))
    assert np.all(np.diff(b) < 0)
