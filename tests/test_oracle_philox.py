"""Pins for the oracle's Philox4x64-10 generator and uniform streams.

numpy.random.Philox is an independent implementation of the same generator
(Salmon et al., SC'11).  Its convention, recorded here: the stored counter is
incremented *before* a block is produced, so the first four words of
Philox(key, counter=c) are the block function at counter c + 1, and
random_raw returns the block's words in order 0..3.
"""
import numpy as np
import pytest

from oracle import philox


def _numpy_block(key, ctr):
    c = [int(x) for x in ctr]
    # step the 256-bit counter back by one (with borrow) for numpy's pre-increment
    for i in range(4):
        if c[i] > 0:
            c[i] -= 1
            break
        c[i] = (1 << 64) - 1
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(c, dtype=np.uint64))
    return [int(x) for x in bg.random_raw(4)]


@pytest.mark.parametrize("key,ctr", [
    ((0, 0), (1, 0, 0, 0)),
    ((5, 7), (1, 0, 0, 0)),
    ((0xFFFFFFFFFFFFFFFF, 0x0123456789ABCDEF), (3, 9, 0, 2)),
    ((2024, 3), (0, 517, 0, 1)),
    ((1, 2), (0xFFFFFFFFFFFFFFFF, 0xFFFFFFFFFFFFFFFF, 7, 0xFFFFFFFFFFFFFFFF)),
])
def test_block_matches_numpy(key, ctr):
    ours = philox.philox4x64_10([np.uint64(c) for c in ctr], [np.uint64(k) for k in key])
    assert [int(w) for w in ours] == _numpy_block(key, ctr)


def test_block_vectorised_matches_numpy():
    rng = np.random.default_rng(0)
    keys = rng.integers(0, 2**63, size=(20, 2), dtype=np.uint64)
    ctrs = rng.integers(0, 2**63, size=(20, 4), dtype=np.uint64)
    ctrs[:, 0] |= np.uint64(1)
    w = philox.philox4x64_10([ctrs[:, i] for i in range(4)], [keys[:, 0], keys[:, 1]])
    for i in range(20):
        assert [int(x[i]) for x in w] == _numpy_block(keys[i], ctrs[i])


def test_mulhilo_against_python_ints():
    rng = np.random.default_rng(1)
    a = rng.integers(0, 2**64 - 1, size=1000, dtype=np.uint64, endpoint=True)
    b = rng.integers(0, 2**64 - 1, size=1000, dtype=np.uint64, endpoint=True)
    hi, lo = philox.mulhilo64(a, b)
    for i in range(1000):
        p = int(a[i]) * int(b[i])
        assert int(hi[i]) == p >> 64 and int(lo[i]) == p & ((1 << 64) - 1)


def test_uniform_range_and_float32_exact():
    u = philox.stream_uniforms(12345, 0, 77, philox.TARGET, 4096)
    assert u.min() > 0.0 and u.max() < 1.0
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)
    # extremes of the 24-bit grid
    assert philox.words_to_uniform(np.uint64(0)) == 2.0**-24
    assert philox.words_to_uniform(np.uint64(0xFFFFFFFFFFFFFFFF)) == 1.0 - 2.0**-24


def test_stream_layout():
    # vocab entry v uses word v & 3 of the block at counter (v >> 2, pos, 0, purpose)
    seed, b, pos, purpose = 99, 3, 1234, philox.DRAFT
    u = philox.stream_uniforms(seed, b, pos, purpose, 10)
    for v in range(10):
        w = _numpy_block((seed, b), (v >> 2, pos, 0, purpose))[v & 3]
        assert u[v] == ((w >> 41) + 0.5) * 2.0**-23
    assert philox.stream_uniform0(seed, b, pos, philox.ACCEPT) == \
        philox.stream_uniforms(seed, b, pos, philox.ACCEPT, 1)[0]


def test_streams_distinct_and_uniform():
    a = philox.stream_uniforms(1, 0, 10, philox.DRAFT, 1 << 16)
    b = philox.stream_uniforms(1, 0, 10, philox.TARGET, 1 << 16)
    c = philox.stream_uniforms(1, 1, 10, philox.DRAFT, 1 << 16)
    assert not np.array_equal(a, b) and not np.array_equal(a, c)
    from scipy import stats
    assert stats.kstest(a, "uniform").pvalue > 1e-4
