"""Pins of the oracle's undirected mappings (iRPE page, Method, eqs. 19-21; CPU only)."""

import math

import numpy as np
import pytest

from oracle import Spec, attention, num_buckets, piecewise_index
from oracle.undirected import distance_rank, piecewise_index_real, undirected_index

ABG = (1.9, 3.8, 15.2)


def _is_two_squares_fermat(k):
    """Sum-of-two-squares test by Fermat's theorem: every prime = 3 (mod 4) occurs
    to an even power (0 counts: 0 = 0^2 + 0^2)."""
    if k == 0:
        return True
    n, p = k, 2
    while p * p <= n:
        e = 0
        while n % p == 0:
            n //= p
            e += 1
        if p % 4 == 3 and e % 2:
            return False
        p += 1
    return not (n > 1 and n % 4 == 3)


def test_distance_rank_page_list():
    # eq. 21: {0, 1, 1.41, 2, 2.24, ...} are numbered 0, 1, 2, 3, 4
    assert [distance_rank(k) for k in (0, 1, 2, 4, 5)] == [0, 1, 2, 3, 4]
    with pytest.raises(ValueError):
        distance_rank(3)            # 3 is no sum of two squares: sqrt(3) is no offset distance


def test_distance_rank_against_fermat():
    ks = [k for k in range(0, 4000) if _is_two_squares_fermat(k)]
    assert [distance_rank(k) for k in ks] == list(range(len(ks)))


def test_page_example_adjacent_offsets():
    # Method, Quantization: (1, 0) and (1, 1) get different buckets; under the Euclidean
    # mapping their distances 1 and 1.41 round to the same index.
    big = (50.0, 60.0, 100.0)       # alpha above every distance used: the exact region
    assert undirected_index(1, 0, "quantized", *big) != undirected_index(1, 1, "quantized", *big)
    assert undirected_index(1, 0, "euclidean", *big) == undirected_index(1, 1, "euclidean", *big) == 1


@pytest.mark.parametrize("dy,dx,want", [(3, 4, 5), (0, 7, 7), (1, 2, 2), (2, 2, 3), (5, 12, 13), (6, 6, 8)])
def test_euclidean_exact_region(dy, dx, want):
    # below alpha the index is the distance rounded (eqs. 18-20); Pythagorean offsets exactly
    assert undirected_index(dy, dx, "euclidean", 50.0, 60.0, 100.0) == want
    assert undirected_index(dy, dx, "euclidean_rounded", 50.0, 60.0, 100.0) == want


@pytest.mark.parametrize("m", ["euclidean", "euclidean_rounded", "quantized", "quantized_squared"])
def test_undirected_invariants(m):
    h = 4
    prev = -1
    for d in range(0, 40):
        # symmetric in signs and in swapping the axes
        v = undirected_index(d, d // 2, m, *ABG)
        assert v == undirected_index(-d, d // 2, m, *ABG) == undirected_index(d // 2, -d, m, *ABG)
        assert 0 <= v <= h
        # non-decreasing in the distance along an axis, saturating at H
        w = undirected_index(d, 0, m, *ABG)
        assert w >= prev
        prev = w
    assert prev == h


def test_on_an_axis_equals_directed_index():
    # dx = 0: the distance is |dy|, an integer, so the Euclidean maps give the directed
    # index of |dy| (eq. 18, pinned separately); the squared form gives that of dy^2
    for reading in ("capped", "trunc"):
        for dy in range(0, 30):
            g = piecewise_index(dy, *ABG, reading)
            assert undirected_index(dy, 0, "euclidean", *ABG, reading) == g
            assert undirected_index(0, dy, "euclidean_rounded", *ABG, reading) == g
            assert undirected_index(dy, 0, "quantized_squared", *ABG, reading) == piecewise_index(dy * dy, *ABG, reading)
    assert piecewise_index_real(math.sqrt(2.0), *ABG) == 1      # 1.41 rounds to 1 below alpha


def test_undirected_attention_on_a_row_is_symmetric_product():
    # On a 1 x N grid every offset lies on the x axis, so the Euclidean mapping is the
    # Product mapping with a table symmetric in dx: P[H*S + H + d] = T[H + g(|d|)].
    rng = np.random.default_rng(23)
    und = Spec(1, 9, prefix=1, mode="contextual", terms={"k", "q", "v"}, map="euclidean",
               alpha=1.9, beta=3.8, gamma=15.2)
    prod = Spec(1, 9, prefix=1, mode="contextual", terms={"k", "q", "v"}, map="piecewise",
                alpha=1.9, beta=3.8, gamma=15.2)
    h, s, rows = num_buckets(und)
    assert rows == s == 9
    _, s2, nb = num_buckets(prod)
    q, k, v = (rng.standard_normal((2, 2, und.tokens_per_image, 5)) for _ in range(3))
    tabs = {n: rng.standard_normal((1, rows, 5)) for n in ("rq", "rk", "rv")}
    ptabs = {}
    for n, t in tabs.items():
        p = np.zeros((1, nb, 5))
        for dxi in range(-h, h + 1):
            p[0, h * s2 + h + dxi] = t[0, h + abs(dxi)]
        ptabs[n] = p
    o1, l1 = attention(und, q, k, v, **tabs)
    o2, l2 = attention(prod, q, k, v, **ptabs)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1, l2, atol=1e-12)
