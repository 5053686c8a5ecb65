"""Pins the oracle's Philox4x64-10 to numpy's independent implementation.

numpy.random.Philox is the 4x64, 10-round generator of Salmon et al. (SC'11).
Its random_raw() increments the 256-bit counter before producing a block, so
the block for counter c is what numpy returns when started at counter c - 1.
"""
import numpy as np
import pytest

M64 = (1 << 64) - 1


def numpy_block(ctr, key):
    c = ctr[0] | ctr[1] << 64 | ctr[2] << 128 | ctr[3] << 192
    g = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=(c - 1) % (1 << 256))
    return [int(v) for v in g.random_raw(4)]


CASES = [
    ((0, 0, 0, 0), (0, 0)),
    ((0, 0, 0, 0), (12345, 0)),
    ((7, 3, 2, 9), (12345, 678)),
    ((M64, M64, M64, M64), (M64, M64)),
    ((255, 5, 1, 99), (0xDEADBEEF, 0)),
    ((1 << 40, 1, 0, 1 << 33), (42, 0)),
]


@pytest.mark.parametrize("ctr,key", CASES)
def test_philox_block_matches_numpy(oracle, ctr, key):
    assert [int(v) for v in oracle.philox(ctr, key)] == numpy_block(ctr, key)


def test_uniform_is_top24_bits_of_word0(oracle):
    rng = np.random.default_rng(1)
    for _ in range(200):
        seed, row, pos, draw, off = (int(x) for x in rng.integers(0, 2**62, 5))
        row, pos, draw = row % 4096, pos % 17, draw % 3
        w0 = numpy_block((row, pos, draw, off), (seed, 0))[0]
        u = oracle.uniform(seed, row, pos, draw, off)
        assert u == (w0 >> 40) / 2.0**24
        assert 0.0 <= u < 1.0
        assert np.float32(u) == u  # exact in fp32


def test_uniform_mean_and_variance(oracle):
    us = np.array([oracle.uniform(0, r, p, 0, 0) for r in range(2000) for p in range(8)])
    assert abs(us.mean() - 0.5) < 4 * np.sqrt(1 / 12 / us.size)
    assert abs(us.var() - 1 / 12) < 0.01
