"""Integer arithmetic the kernels rely on, checked on the host.

The fused decoding step takes the CAPE digits of a slot with a run-time base
d_p by a multiply-high: x / d = mulhi(x, m) with m = ceil(2^32 / d).  The
kernels use it for slot values x < 2^30 (the largest slot count) and bases
2..8.  Writing x = q d + r, mulhi gives floor(q + r / d + x e / (d 2^32))
with e = m d - 2^32, which equals q whenever x e < 2^32; these tests pin the
bound on e for every base and check the quotient on the values nearest to
where it would first fail (the top of the range, around multiples of d)."""
import numpy as np
import pytest

X_MAX = 1 << 30  # the kernels' slot values are below 2^30


def mulhi_reciprocal(d: int) -> int:
    return (2**32 - 1) // d + 1


@pytest.mark.parametrize("d", range(2, 9))
def test_error_term_keeps_quotient_exact(d):
    m = mulhi_reciprocal(d)
    assert m == -(-(2**32) // d)  # ceil(2^32 / d)
    e = m * d - 2**32
    assert 0 <= e <= 4
    assert (X_MAX - 1) * e < 2**32


@pytest.mark.parametrize("d", range(2, 9))
def test_quotients_near_the_top_and_at_multiples(d):
    m = np.uint64(mulhi_reciprocal(d))
    top = np.arange(X_MAX - 4096, X_MAX, dtype=np.uint64)
    rng = np.random.default_rng(d)
    mult = rng.integers(0, X_MAX // d, 4096, dtype=np.uint64) * np.uint64(d)
    x = np.concatenate([top, mult, mult - np.uint64(1), mult + np.uint64(d - 1),
                        np.arange(0, 4096, dtype=np.uint64)])
    x = x[(x < X_MAX)]
    q = (x * m) >> np.uint64(32)
    assert np.array_equal(q, x // np.uint64(d))
