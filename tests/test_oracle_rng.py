"""Pins for the oracle's counter-based generator, uniform mapping, specified ln, Gumbel."""
import math

import numpy as np
import pytest

from oracle import eagle3_oracle as O

# Known-answer vectors published with the Random123 library for philox4x32 with 10
# rounds (counter words c0..c3, key words k0, k1 -> four output words).
KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,expect", KAT)
def test_philox_known_answers(ctr, key, expect):
    out = O.philox4x32_10(*ctr, *key)
    assert tuple(int(np.asarray(w)) for w in out) == expect


def test_philox_vectorised_matches_scalar():
    c = np.arange(50, dtype=np.uint64) * np.uint64(0x9E3779B1)
    v = O.philox4x32_10(c, c + 1, c + 2, c + 3, 7, 9)
    for n in range(0, 50, 7):
        s = O.philox4x32_10(int(c[n]) & 0xFFFFFFFF, (int(c[n]) + 1) & 0xFFFFFFFF,
                            (int(c[n]) + 2) & 0xFFFFFFFF, (int(c[n]) + 3) & 0xFFFFFFFF, 7, 9)
        assert tuple(int(x[n]) for x in v) == tuple(int(x) for x in s)


def test_uniform23_range_and_exactness():
    u = O.uniform23(np.array([0, 511, 512, 0xFFFFFFFF], dtype=np.uint64))
    assert u.dtype == np.float32
    assert float(u[0]) == 2.0 ** -24 and float(u[1]) == 2.0 ** -24
    assert float(u[2]) == 1.5 * 2.0 ** -23
    assert float(u[3]) == 1.0 - 2.0 ** -24
    assert np.all((u > 0) & (u < 1))
    # every cell centre is exact: u * 2^23 - 0.5 recovers the integer
    x = np.random.default_rng(0).integers(0, 2**32, 100000, dtype=np.uint64)
    back = O.uniform23(x).astype(np.float64) * 2.0 ** 23 - 0.5
    assert np.array_equal(back, (x >> np.uint64(9)).astype(np.float64))


def ulp32(x):
    x = np.abs(np.asarray(x, dtype=np.float32))
    return np.spacing(x).astype(np.float64)


def test_ln_spec_accuracy():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        np.float32(2.0) ** rng.uniform(-26, 5, 200000).astype(np.float32),
        np.array([1.0, 2.0, 0.5, 1.41421354, 1.41421342, 0.70710677, 3e-8, 17.3], np.float32),
    ]).astype(np.float32)
    got = O.ln_spec(v).astype(np.float64)
    ref = np.log(v.astype(np.float64))
    err = np.abs(got - ref) / np.maximum(ulp32(ref), 2.0 ** -149)
    assert float(np.max(err)) <= 2.0
    assert float(O.ln_spec(np.float32(1.0))) == 0.0
    assert float(O.ln_spec(np.float32(2.0))) == float(np.float32(math.log(2.0)))


def test_gumbel_moments_and_determinism():
    t = np.arange(1 << 20)
    g = O.gumbel(1234, 5, 0, 3, t).astype(np.float64)
    # standard Gumbel: mean = Euler-Mascheroni gamma, variance = pi^2 / 6
    assert abs(g.mean() - 0.5772156649) < 5e-3
    assert abs(g.var() - math.pi ** 2 / 6) < 2e-2
    assert np.array_equal(O.gumbel(1234, 5, 0, 3, t[:1000]), g[:1000].astype(np.float32))
    assert not np.array_equal(O.gumbel(1234, 6, 0, 3, t[:1000]), g[:1000].astype(np.float32))
    # the 24-bit uniforms bound the noise
    assert g.max() < 16.7 and g.min() > -2.9
