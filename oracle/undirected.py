"""Undirected bucket indices of a 2D offset (oracle, fp64).

Test infrastructure only (see the package docstring).

Source: iRPE summary page ("Rethinking and Improving Relative Position
Encoding for Vision Transformer"), Method, the Euclidean mapping (eqs. 19-20)
and the Quantization mapping (eq. 21), and "Paper vs code" for how the
released code differs.  Both are undirected: the index of (dy, dx) depends on
the distance of the offset only, so it is never negative and a table of
S = 2H+1 rows (H as for eq. 18) is indexed by index + H.

Four maps, two per mapping:

``euclidean``          the index function of eq. 18 applied to the real
                       distance r = sqrt(dy^2 + dx^2) (eqs. 19-20): r <= alpha
                       keeps its rounded value, beyond alpha the log-spaced
                       position of r is capped and rounded as for an integer
                       offset (the reading of eq. 18 is shared).
``euclidean_rounded``  the code's order: the distance is rounded to an integer
                       first, then eq. 18 applies ("Paper vs code", Euclidean
                       rounding order).
``quantized``          eq. 21: the distances that integer offsets can have,
                       {0, 1, 1.41, 2, 2.24, ...} = sqrt of the integers that
                       are sums of two squares, are numbered 0, 1, 2, ... in
                       increasing order, and eq. 18 applies to that number.
                       The numbering runs over all integer offsets, not only
                       those of one unit.
``quantized_squared``  the code's form: eq. 18 applied to the squared distance
                       dy^2 + dx^2 ("Paper vs code", Quantization mapping).
"""

import math
from functools import lru_cache

from .index import ROUND_CAPPED, ROUND_TRUNC, _check_params, log_position, piecewise_index, round_half_away

UNDIRECTED_MAPS = ("euclidean", "euclidean_rounded", "quantized", "quantized_squared")


def piecewise_index_real(r, alpha, beta, gamma, reading=ROUND_CAPPED):
    """Eq. 18 for a real r >= 0 (the distance of an offset)."""
    _check_params(alpha, beta, gamma)
    if r < 0:
        raise ValueError("a distance is never negative")
    if r <= alpha:
        return int(round_half_away(r))
    s = log_position(r, alpha, beta, gamma)
    if reading == ROUND_CAPPED:
        return int(round_half_away(min(beta, round_half_away(s))))
    if reading == ROUND_TRUNC:
        return int(math.trunc(min(beta, round_half_away(s))))
    raise ValueError(f"unknown reading {reading!r}")


@lru_cache(maxsize=None)
def _two_square_sums(limit):
    """Sorted integers m <= limit with m = a^2 + b^2 for integers a, b >= 0."""
    found = set()
    a = 0
    while a * a <= limit:
        b = a
        while a * a + b * b <= limit:
            found.add(a * a + b * b)
            b += 1
        a += 1
    return tuple(sorted(found))


def distance_rank(k):
    """Position of sqrt(k) among the distances integer offsets can have (eq. 21):
    the number of sums of two squares smaller than k.  k must be one itself."""
    sums = _two_square_sums(k)
    if sums[-1] != k:
        raise ValueError(f"{k} is not a sum of two squares")
    return len(sums) - 1


def undirected_index(dy, dx, map, alpha, beta, gamma, reading=ROUND_CAPPED):
    """Index in [0, H] of the offset (dy, dx) under one of the undirected maps."""
    k = int(dy) * int(dy) + int(dx) * int(dx)
    if map == "euclidean":
        return piecewise_index_real(math.sqrt(k), alpha, beta, gamma, reading)
    if map == "euclidean_rounded":
        return piecewise_index(int(round_half_away(math.sqrt(k))), alpha, beta, gamma, reading)
    if map == "quantized":
        return piecewise_index(distance_rank(k), alpha, beta, gamma, reading)
    if map == "quantized_squared":
        return piecewise_index(k, alpha, beta, gamma, reading)
    raise ValueError(f"map {map!r} is not undirected")
