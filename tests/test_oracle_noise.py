"""Pins of the oracle's noise: Philox against an independent implementation,
uniforms and Gumbel values against exact / high-precision arithmetic, and the
Gumbel moments against their closed forms."""
import decimal
import math
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

from oracle import philox4x32_10, noise_words, uniform24, gumbel, SALT_DRAFT
from oracle.noise import SALT_ACCEPT, SALT_RESAMPLE

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_kat(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND reference")
    exe = str(tmp_path_factory.mktemp("kat") / "kat")
    subprocess.run([hipcc, "-O1", "-o", exe, os.path.join(HERE, "support", "rocrand_philox_kat.cpp")], check=True,
                   capture_output=True)

    def run(seed, subseq, offset, n):
        out = subprocess.run([exe, str(seed), str(subseq), str(offset), str(n)], check=True, capture_output=True,
                             text=True).stdout.split()
        return np.array([int(w, 16) for w in out], dtype=np.uint32)

    return run


@pytest.mark.parametrize("seed,subseq,offset", [
    (0, 0, 0),
    (123, 5, 0),
    (0xFFFFFFFFFFFFFFFF, 0xFFFFFFFFFFFFFFFF, 0),
    (0x0123456789ABCDEF, 0xDEADBEEF00C0FFEE, 4 * 77),
    (42, 7, 4 * 0xFFFFFFFE),  # the counter's low word carries into word 1
])
def test_philox_matches_rocrand(rocrand_kat, seed, subseq, offset):
    n = 16
    ref = rocrand_kat(seed, subseq, offset, n)
    ctr = offset // 4 + np.arange(n // 4, dtype=object)
    got = []
    for c in ctr:
        c = int(c)
        w = philox4x32_10(c & 0xFFFFFFFF, c >> 32, subseq & 0xFFFFFFFF, subseq >> 32, seed & 0xFFFFFFFF, seed >> 32)
        got.extend(int(x) for x in w)
    assert np.array_equal(np.array(got, dtype=np.uint32), ref)


@pytest.mark.parametrize("salt", [SALT_DRAFT, SALT_ACCEPT, SALT_RESAMPLE])
def test_noise_word_layout_matches_rocrand(rocrand_kat, salt):
    # Column c of the draw keyed (seed, pos, salt) is word c&3 of counter
    # (c>>2, pos_lo, pos_hi, salt). In rocRAND's terms: offset counter
    # (pos_lo << 32 | c>>2) and subsequence (salt << 32 | pos_hi).
    seed = 0x1234_5678_9ABC_DEF0
    pos = (3 << 32) | 0x0BADF00D
    cols = np.arange(64)
    got = noise_words(seed, pos, salt, cols)
    subseq = (salt << 32) | (pos >> 32)
    offset = 4 * ((pos & 0xFFFFFFFF) << 32)
    ref = rocrand_kat(seed, subseq, offset, 64)
    assert np.array_equal(got, ref)


def test_negative_seed_is_twos_complement():
    a = noise_words(-1, 5, SALT_DRAFT, np.arange(8))
    b = noise_words(0xFFFFFFFFFFFFFFFF - 2**64 + 2**64, 5, SALT_DRAFT, np.arange(8))
    c = philox4x32_10(np.arange(2), 5, 0, SALT_DRAFT, 0xFFFFFFFF, 0xFFFFFFFF)
    assert np.array_equal(a, b)
    assert np.array_equal(a, np.stack(c, -1).reshape(-1))


def test_uniform_values_are_odd_multiples_inside_unit_interval():
    w = np.array([0, 1, 511, 512, 0x80000000, 0xFFFFFE00, 0xFFFFFFFF], dtype=np.uint32)
    u = uniform24(w)
    k = u * 2**24
    assert np.all(k == np.round(k)) and np.all(k.astype(np.int64) % 2 == 1)
    assert u[0] == 2.0**-24 and u[-1] == 1 - 2.0**-24
    assert np.all((u > 0) & (u < 1))
    assert np.all(u.astype(np.float32).astype(np.float64) == u)  # exact in float32
    # symmetric around 1/2: word w and its complement give u and 1-u
    rng = np.random.default_rng(0)
    ww = rng.integers(0, 2**32, 1000, dtype=np.uint64).astype(np.uint32)
    assert np.allclose(uniform24(ww) + uniform24(~ww), 1.0, rtol=0, atol=0)


def _gumbel_decimal(u: float) -> float:
    with decimal.localcontext() as ctx:
        ctx.prec = 60
        d = decimal.Decimal(u)  # exact binary value
        return float(-((-(d.ln())).ln()))


@pytest.mark.parametrize("u", [2.0**-24, 3 * 2.0**-24, 0.25, 0.5, 0.75, math.exp(-1) // 2**-24 * 2**-24 + 2**-24,
                               1 - 3 * 2.0**-24, 1 - 2.0**-24])
def test_gumbel_matches_high_precision(u):
    ref = _gumbel_decimal(u)
    got = float(gumbel(np.array([u]))[0])
    assert abs(got - ref) <= 4e-16 * max(1.0, abs(ref))


def test_gumbel_extremes_closed_form():
    # u = 1 - 2**-24: -log u = 2**-24 (1 + 2**-25 + ...), g = 24 log 2 - log1p(~2**-25)
    g = float(gumbel(np.array([1 - 2.0**-24]))[0])
    assert abs(g - (24 * math.log(2) - 2.0**-25)) < 1e-12
    assert abs(g - 16.6355323) < 1e-6


def test_uniform_and_gumbel_moments():
    n = 1 << 20
    w = noise_words(987654321, 1000, SALT_DRAFT, np.arange(n))
    u = uniform24(w)
    assert abs(u.mean() - 0.5) < 5 * math.sqrt(1 / 12 / n)
    assert abs(u.var() - 1 / 12) < 5 * math.sqrt(1 / 180 / n)
    assert stats.kstest(u, "uniform").pvalue > 1e-4
    g = gumbel(u)
    euler_gamma = 0.5772156649015329
    var = math.pi**2 / 6
    assert abs(g.mean() - euler_gamma) < 5 * math.sqrt(var / n)
    # fourth central moment of the standard Gumbel is 27/5 * var**2
    assert abs(g.var() - var) < 5 * math.sqrt((27 / 5 - 1) * var**2 / n)
    assert stats.kstest(g, "gumbel_r").pvalue > 1e-4


def test_streams_differ_by_salt_and_position():
    cols = np.arange(4096)
    a = noise_words(7, 100, SALT_DRAFT, cols)
    assert not np.array_equal(a, noise_words(7, 100, SALT_RESAMPLE, cols))
    assert not np.array_equal(a, noise_words(7, 101, SALT_DRAFT, cols))
    assert not np.array_equal(a, noise_words(8, 100, SALT_DRAFT, cols))
    # words of adjacent positions are uncorrelated
    r = np.corrcoef(uniform24(a), uniform24(noise_words(7, 101, SALT_DRAFT, cols)))[0, 1]
    assert abs(r) < 5 / math.sqrt(cols.size)
