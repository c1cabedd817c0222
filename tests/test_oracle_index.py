"""Pins of the oracle's per-axis index function and bucket ids (CPU only).

Each pin comes from outside the oracle: a value printed on the pages, a count
stated by the workload definitions, or an invariant the pages state.
"""

import itertools
import math
import os

import numpy as np
import pytest

from oracle import (ROUND_CAPPED, ROUND_TRUNC, Spec, axis_index_table, bucket_map,
                    half_width, num_buckets, piecewise_index, round_half_away)
from oracle.attention import bucket_map_array

PARAMS = [(1.9, 3.8, 15.2), (3.8, 7.6, 30.4), (2.0, 4.0, 16.0), (1.0, 2.0, 8.0),
          (3.0, 3.0, 8.0), (2.5, 6.3, 21.7), (0.5, 1.6, 5.0)]


def _read(path):
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_round_half_away():
    assert round_half_away(2.5) == 3 and round_half_away(-2.5) == -3
    assert round_half_away(2.49) == 2 and round_half_away(-0.5) == -1
    assert round_half_away(0.0) == 0


@pytest.mark.parametrize("reading", [ROUND_CAPPED, ROUND_TRUNC])
@pytest.mark.parametrize("abg", PARAMS)
def test_exact_for_small_offsets(abg, reading):
    # iRPE page, Method, eq. 18: offsets up to alpha keep their own integer index.
    a, b, g = abg
    for x in range(-int(math.floor(a)), int(math.floor(a)) + 1):
        assert piecewise_index(x, a, b, g, reading) == x


@pytest.mark.parametrize("reading", [ROUND_CAPPED, ROUND_TRUNC])
@pytest.mark.parametrize("abg", PARAMS)
def test_odd_monotone_saturating(abg, reading):
    # eq. 18: the sign is kept (odd), the index grows with |x| and is capped at beta,
    # so it saturates at the table half-width.
    a, b, g = abg
    h = half_width(a, b, g, reading)
    vals = [piecewise_index(x, a, b, g, reading) for x in range(0, 400)]
    for x in range(0, 400):
        assert piecewise_index(-x, a, b, g, reading) == -vals[x]
    assert all(v2 >= v1 for v1, v2 in zip(vals, vals[1:]))
    assert max(vals) == h and vals[-1] == h
    assert all(abs(v) <= b + 0.5 for v in vals)


def test_trunc_partition_page_example(golden_dir):
    # iRPE page, Pitfalls "Bucket edges are sharp": hand-worked partition at r = 1.9.
    for off, idx in _read(os.path.join(golden_dir, "irpe_partition_trunc_r1.9.txt")):
        assert piecewise_index(int(off), 1.9, 3.8, 15.2, ROUND_TRUNC) == int(idx)


def test_trunc_r2_shares_2_and_3():
    # iRPE page, Pitfalls: with r = 2.0 offsets 2 and 3 also share a bucket.
    g = [piecewise_index(x, 2.0, 4.0, 16.0, ROUND_TRUNC) for x in range(5)]
    assert g[2] == g[3] and g[1] != g[2]


def test_bucket_counts(golden_dir):
    # Reachable per-axis index values on the workload grids, and the Product table size.
    for reading, a, b, g, side, per_axis, total in _read(os.path.join(golden_dir, "bucket_counts.txt")):
        a, b, g, side, per_axis, total = float(a), float(b), float(g), int(side), int(per_axis), int(total)
        vals = set(axis_index_table(side, a, b, g, reading))
        assert len(vals) == per_axis
        h = half_width(a, b, g, reading)
        assert 2 * h + 1 == per_axis
        spec = Spec(side, side, mode="contextual", terms={"k"}, map="piecewise",
                    alpha=a, beta=b, gamma=g, reading=reading)
        assert num_buckets(spec)[2] == total
        ids = set(bucket_map_array(spec).ravel().tolist())
        assert len(ids) == total and min(ids) == 0 and max(ids) == total - 1


def test_no_rounding_tie_at_workload_grids():
    # The tie rule is not fixed by the pages; at the workload parameters no offset
    # lands within 1e-3 of a tie, so any tie rule gives the same indices.
    from oracle.index import log_position
    for a, b, g, side in [(1.9, 3.8, 15.2, 14), (3.8, 7.6, 30.4, 56)]:
        for x in range(int(a) + 1, side):
            s = log_position(x, a, b, g)
            assert abs((s - math.floor(s)) - 0.5) > 1e-3


def test_readings_differ_only_far_out():
    # The two readings agree up to offset 10 at r = 1.9 and up to 28 at r = 3.8.
    for (a, b, g), last_same in [((1.9, 3.8, 15.2), 10), ((3.8, 7.6, 30.4), 28)]:
        ca = [piecewise_index(x, a, b, g, ROUND_CAPPED) for x in range(0, 60)]
        tr = [piecewise_index(x, a, b, g, ROUND_TRUNC) for x in range(0, 60)]
        assert ca[:last_same + 1] == tr[:last_same + 1]
        assert ca[last_same + 1] == tr[last_same + 1] + 1


def test_clip_special_case():
    # alpha = beta = k gives the clip function of prior 1D methods (iRPE page, Method,
    # prior 1D methods: distances beyond k share one vector).
    for k in (1, 2, 3, 5):
        for x in range(-20, 21):
            assert piecewise_index(x, k, k, k + 7.5) == max(-k, min(k, x))


def test_swin_worked_example(golden_dir):
    # Swin post, section 3.2: M = 3, (0,0) -> (2,2) has offset (-2,-2) -> cell (0,0) of 5x5.
    (m, qr, qc, kr, kc, oy, ox, cy, cx, side), = [list(map(int, r)) for r in
                                                  _read(os.path.join(golden_dir, "swin_m3_example.txt"))]
    spec = Spec(m, m, window=m, mode="bias", map="swin")
    h, s, nb = num_buckets(spec)
    assert s == side and nb == side * side
    bm = bucket_map(spec)
    qi, ki = qr * m + qc, kr * m + kc
    assert (qr - kr, qc - kc) == (oy, ox)
    assert bm[qi][ki] == cy * side + cx == 0
    # and the opposite pair lands in the opposite corner
    assert bm[ki][qi] == side * side - 1


def test_swin_table_sizes(golden_dir):
    # Swin post, section 3.3.
    for m, direct, side, compact in [list(map(int, r)) for r in
                                     _read(os.path.join(golden_dir, "swin_table_sizes.txt"))]:
        spec = Spec(m, m, window=m, mode="bias", map="swin")
        h, s, nb = num_buckets(spec)
        assert (s, nb) == (side, compact)
        bm = bucket_map_array(spec)
        assert bm.size == direct
        assert len(set(bm.ravel().tolist())) == compact


@pytest.mark.parametrize("spec", [
    Spec(4, 5, mode="contextual", terms={"k"}, map="piecewise", alpha=1.9, beta=3.8, gamma=15.2),
    Spec(6, 6, mode="contextual", terms={"k"}, map="piecewise", alpha=1.0, beta=2.0, gamma=8.0,
         reading=ROUND_TRUNC, prefix=1),
    Spec(6, 4, window=2, mode="bias", map="swin"),
    Spec(5, 5, mode="bias", map="swin"),
])
def test_translation_invariance_and_scalar_vs_vector(spec):
    # Swin post, section 2.2: pairs with the same offset share one entry.  The scalar
    # per-pair definition and the vectorised map must agree.
    from oracle import unit_positions
    for u in range(spec.units_per_image):
        toks = unit_positions(spec, u)
        bm = np.array(bucket_map(spec, u))
        assert (bm == bucket_map_array(spec, u)).all()
        by_offset = {}
        for (i, (_, pi)), (j, (_, pj)) in itertools.product(enumerate(toks), enumerate(toks)):
            if pi is None or pj is None:
                assert bm[i, j] == -1
                continue
            off = (pi[0] - pj[0], pi[1] - pj[1])
            by_offset.setdefault(off, set()).add(int(bm[i, j]))
        assert all(len(v) == 1 for v in by_offset.values())
        if spec.map == "swin":
            # distinct offsets get distinct cells (the compact table is exact)
            assert len({next(iter(v)) for v in by_offset.values()}) == len(by_offset)


def test_swin_is_product_special_case():
    # Swin map = Product map with every offset exact (alpha >= M-1) and beta = M-1.
    for m in (2, 3, 4, 7):
        sw = Spec(m, m, window=m, mode="bias", map="swin")
        pr = Spec(m, m, mode="contextual", terms={"k"}, map="piecewise",
                  alpha=m - 1 + 0.5 if m > 1 else 0.5, beta=m - 1 + 0.5, gamma=4.0 * m,
                  reading=ROUND_TRUNC)
        assert (bucket_map_array(sw) == bucket_map_array(pr)).all()


def test_axis_order_rows_first():
    # iRPE page, Method, Product bucket pseudo-code: id = (row index + H) * S + (col index + H).
    spec = Spec(3, 3, window=3, mode="bias", map="swin")
    bm = bucket_map_array(spec)
    # query (0,0), key (0,2): offset (0,-2) -> row cell 2, col cell 0 -> id 10
    assert bm[0, 2] == 2 * 5 + 0
    # query (0,0), key (2,0): offset (-2,0) -> row cell 0, col cell 2 -> id 2
    assert bm[0, 6] == 0 * 5 + 2


def test_bad_params_rejected():
    for a, b, g in [(0.0, 3.0, 8.0), (2.0, 1.0, 8.0), (2.0, 3.0, 2.0), (-1.0, 3.0, 8.0)]:
        with pytest.raises(ValueError):
            piecewise_index(5, a, b, g)
    with pytest.raises(ValueError):
        Spec(4, 4, window=3)
    with pytest.raises(ValueError):
        Spec(4, 4, mode="bias", terms={"v"})


@pytest.mark.parametrize("reading", [ROUND_CAPPED, ROUND_TRUNC])
@pytest.mark.parametrize("abg", PARAMS)
def test_step_positions_closed_form(abg, reading):
    # Where each step of g lies, from the inverse of eq. 18 rather than from
    # evaluating it.  The page's index grows like log(|x|/alpha)/log(gamma/alpha),
    # scaled to reach beta at gamma, and is rounded; so beyond alpha the index
    # reaches k exactly where the real position passes k - 1/2, i.e. at the first
    # integer offset a > alpha with
    #     a >= alpha * (gamma/alpha) ** ((k - 1/2 - alpha) / (beta - alpha)),
    # for every k up to the table half-width (the cap at beta only stops the
    # count there: capped, H = rh(beta); truncating, H = trunc(beta)).  Inside
    # |x| <= alpha the index is the offset.  This places every step of both
    # readings, the capped reading's last one included (offsets 11 at r = 1.9 and
    # 29 at r = 3.8), with an exponential instead of the oracle's logarithm.
    a, b, g = abg
    h = half_width(a, b, g, reading)
    thresholds = []
    for k in range(1, h + 1):
        if k <= math.floor(a):
            thresholds.append(k)
            continue
        if b == a:
            edge = 0.0                      # the real position is alpha everywhere beyond alpha
        else:
            edge = a * (g / a) ** ((k - 0.5 - a) / (b - a))
            frac = edge - math.floor(edge)
            assert min(frac, 1 - frac) > 1e-9, "an offset sits on a rounding edge"
        thresholds.append(max(math.floor(a) + 1, math.ceil(edge)))
    for x in range(0, 400):
        want = sum(1 for t in thresholds if t <= x)
        assert piecewise_index(x, a, b, g, reading) == want, (x, thresholds)
        assert piecewise_index(-x, a, b, g, reading) == -want
    if abg == (1.9, 3.8, 15.2) and reading == ROUND_CAPPED:
        assert thresholds == [1, 2, 4, 11]
    if abg == (3.8, 7.6, 30.4) and reading == ROUND_CAPPED:
        assert thresholds[-1] == 29
