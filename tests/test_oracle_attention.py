"""Pins of the oracle's attention forward (CPU only).

The oracle is pinned to things outside itself: a library softmax attention
(torch fp64 on the CPU) for the cases the method reduces to plain attention,
printed weights from the Shaw-style page, the Swin worked example turned into
an attention pattern, and a pure-loop implementation on tiny shapes.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import Spec, attention, attention_literal, num_buckets, unit_token_indices
from oracle.attention import bucket_map_array


def sdpa(q, k, v, scale):
    """Library softmax attention in float64 on the CPU, [B, H, T, d]."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=scale).numpy()


def _rand(rng, *shape, sigma=1.0):
    return sigma * rng.standard_normal(shape)


def _inputs(spec, B, H, d, rng, sigma=1.0, per_head=False):
    N = spec.tokens_per_image
    q, k, v = (_rand(rng, B, H, N, d) for _ in range(3))
    _, _, nb = num_buckets(spec)
    th = H if per_head else 1
    tabs = {}
    if spec.mode == "bias":
        tabs["bias"] = _rand(rng, th, nb, sigma=sigma)
    if spec.mode == "contextual":
        for t in sorted(spec.terms):
            tabs["r" + t] = _rand(rng, th, nb, d, sigma=sigma)
    return q, k, v, tabs


TINY = [
    Spec(2, 3, mode="contextual", terms={"k"}, map="piecewise", alpha=1.0, beta=2.0, gamma=8.0),
    Spec(3, 3, prefix=1, mode="contextual", terms={"k", "q", "v"}, map="piecewise",
         alpha=0.9, beta=1.7, gamma=3.0),
    Spec(1, 6, mode="contextual", terms={"q", "v"}, map="piecewise", alpha=1.5, beta=2.5,
         gamma=4.0, reading="trunc"),
    Spec(4, 4, window=2, mode="bias", map="swin"),
    Spec(4, 4, prefix=1, mode="bias", map="piecewise", alpha=1.0, beta=2.0, gamma=4.0),
    Spec(3, 2, mode="none"),
]


@pytest.mark.parametrize("spec", TINY)
@pytest.mark.parametrize("per_head", [False, True])
def test_literal_matches_vectorised(spec, per_head):
    rng = np.random.default_rng(7)
    q, k, v, tabs = _inputs(spec, 2, 2, 5, rng, per_head=per_head)
    o1, l1 = attention_literal(spec, q, k, v, **tabs)
    o2, l2 = attention(spec, q, k, v, **tabs)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)


@pytest.mark.parametrize("spec", [
    Spec(4, 4, window=4, mode="bias", map="swin"),
    Spec(6, 6, window=3, mode="bias", map="swin"),
    Spec(5, 4, prefix=1, mode="contextual", terms={"k", "q", "v"}, map="piecewise",
         alpha=1.9, beta=3.8, gamma=15.2),
    Spec(7, 7, mode="none"),
])
def test_zero_tables_give_plain_attention(spec):
    # Tables start at zero (iRPE page, supp. Weight Initialization); with zero tables
    # the method is plain softmax attention (eqs. 1-3).
    rng = np.random.default_rng(11)
    B, H, d = 2, 3, 8
    q, k, v, tabs = _inputs(spec, B, H, d, rng)
    tabs = {n: np.zeros_like(t) for n, t in tabs.items()}
    o, lse = attention(spec, q, k, v, **tabs)
    s = 1 / math.sqrt(d)
    for u in range(spec.units_per_image):
        idx = unit_token_indices(spec, u)
        ref = sdpa(q[:, :, idx], k[:, :, idx], v[:, :, idx], s)
        np.testing.assert_allclose(o[:, :, idx], ref, rtol=0, atol=1e-12)
        lg = np.einsum("bhid,bhjd->bhij", q[:, :, idx], k[:, :, idx]) * s
        ref_lse = torch.logsumexp(torch.from_numpy(lg), dim=-1).numpy()
        np.testing.assert_allclose(lse[:, :, idx], ref_lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("prefix", [0, 1])
def test_constant_tables_closed_forms(prefix):
    # With every table row equal to one vector u the position terms become content terms:
    #   rK = u  -> q.(k_j + u):  plain attention with keys k + u   (eq. 15)
    #   rQ = u  -> k_j.(q_i + u): plain attention with queries q + u (eq. 16)
    #   rV = w  -> every output gains w, since the weights sum to 1   (eq. 17)
    # Prefix pairs receive none of these terms.
    spec = Spec(4, 3, prefix=prefix, mode="contextual", terms={"k", "q", "v"}, map="piecewise",
                alpha=1.0, beta=2.0, gamma=6.0)
    rng = np.random.default_rng(5)
    B, H, d = 2, 2, 6
    N = spec.tokens_per_image
    q, k, v, _ = _inputs(spec, B, H, d, rng)
    _, _, nb = num_buckets(spec)
    uk, uq, w = rng.standard_normal(d), rng.standard_normal(d), rng.standard_normal(d)
    s = 1 / math.sqrt(d)
    zero = np.zeros((1, nb, d))

    o, _ = attention(spec, q, k, v, rk=np.tile(uk, (1, nb, 1)), rq=zero, rv=zero)
    kk = k + uk
    kk[:, :, :prefix] = k[:, :, :prefix]
    ref = sdpa(q, kk, v, s)
    if prefix:
        ref[:, :, :prefix] = sdpa(q[:, :, :prefix], k, v, s)
        # a positioned query sees the prefix key without the shift: handled by logits below
        lg = np.einsum("bhid,bhjd->bhij", q, kk) * s
        lg[:, :, :prefix, :] = np.einsum("bhid,bhjd->bhij", q[:, :, :prefix], k) * s
        a = torch.softmax(torch.from_numpy(lg), -1).numpy()
        ref = a @ v
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)

    o, _ = attention(spec, q, k, v, rk=zero, rq=np.tile(uq, (1, nb, 1)), rv=zero)
    lg = np.einsum("bhid,bhjd->bhij", q + uq, k) * s
    if prefix:
        plain = np.einsum("bhid,bhjd->bhij", q, k) * s
        lg[:, :, :prefix, :] = plain[:, :, :prefix, :]
        lg[:, :, :, :prefix] = plain[:, :, :, :prefix]
    a = torch.softmax(torch.from_numpy(lg), -1).numpy()
    np.testing.assert_allclose(o, a @ v, rtol=0, atol=1e-12)

    o, _ = attention(spec, q, k, v, rk=zero, rq=zero, rv=np.tile(w, (1, nb, 1)))
    lg = np.einsum("bhid,bhjd->bhij", q, k) * s
    a = torch.softmax(torch.from_numpy(lg), -1).numpy()
    ref = a @ v
    if prefix:
        # rows of positioned queries gain w times the weight on positioned keys
        ref = ref + a[:, :, :, prefix:].sum(-1, keepdims=True) * w
        ref[:, :, :prefix] = (a @ v)[:, :, :prefix]
    else:
        ref = ref + w
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_constant_bias_is_softmax_invariant():
    spec = Spec(6, 6, window=3, mode="bias", map="swin")
    rng = np.random.default_rng(3)
    q, k, v, tabs = _inputs(spec, 1, 2, 4, rng)
    o0, _ = attention(spec, q, k, v, bias=np.zeros_like(tabs["bias"]))
    o1, _ = attention(spec, q, k, v, bias=np.full_like(tabs["bias"], 3.25))
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-12)


def test_swin_example_as_attention():
    # Swin post, section 3.2 worked example, M = 3: only the pair query (0,0) -> key (2,2)
    # has offset (-2,-2), stored in cell (0,0) = flat id 0.  A large bias in that cell alone
    # makes query 0 attend to key 8 and no other query change.  A sign or transposition
    # error would move the attention to query 8 -> key 0 instead.
    spec = Spec(3, 3, window=3, mode="bias", map="swin")
    rng = np.random.default_rng(9)
    q, k, v = (0.1 * rng.standard_normal((1, 1, 9, 4)) for _ in range(3))
    bias = np.zeros((1, 25))
    bias[0, 0] = 60.0
    o, _, wts = attention(spec, q, k, v, bias=bias, return_weights=True)
    a = wts[(0, 0, 0)]
    assert a[0, 8] > 0.999999
    assert (a[1:, 8] < 0.5).all()
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 8], atol=1e-6)


def test_axis_order_as_attention():
    # Row offsets index the table's rows: a bias at cell [dy + 3][dx + 3] with (dy, dx) =
    # (-2, 0) on a 4x4 window (7x7 table) reaches exactly the pairs two rows apart in the
    # same column, query above key.
    spec = Spec(4, 4, window=4, mode="bias", map="swin")
    bias = np.zeros((1, 49))
    bias[0, (-2 + 3) * 7 + (0 + 3)] = 60.0
    rng = np.random.default_rng(2)
    q, k, v = (0.1 * rng.standard_normal((1, 1, 16, 4)) for _ in range(3))
    _, _, wts = attention(spec, q, k, v, bias=bias, return_weights=True)
    a = wts[(0, 0, 0)]
    for i in range(16):
        r, c = divmod(i, 4)
        if r + 2 < 4:
            assert a[i, (r + 2) * 4 + c] > 0.999999
        else:
            assert a[i].max() < 0.5


def _shaw_page_setup():
    """Inputs of the Shaw-style page's test run, drawn as that page describes.

    Input X (6 x 8) after seeding NumPy's legacy generator with 42; then, after
    reseeding with 123, the three 8 x 4 projections for q, k, v, each scaled by
    sqrt(2 / (8 + 4)); then, after reseeding with 123 again, the key and value
    relative tables (7 offsets x 4) scaled by sqrt(2 / (7 + 4)).
    """
    rs = np.random.RandomState(42)
    x = rs.randn(6, 8)
    rs = np.random.RandomState(123)
    sc = math.sqrt(2.0 / 12.0)
    wq, wk, wv = rs.randn(8, 4) * sc, rs.randn(8, 4) * sc, rs.randn(8, 4) * sc
    rs = np.random.RandomState(123)
    st = math.sqrt(2.0 / 11.0)
    a_k, a_v = rs.randn(7, 4) * st, rs.randn(7, 4) * st
    return x @ wq, x @ wk, x @ wv, a_k, a_v


def _shaw_as_2d(a_k, a_v, mirror=True):
    """The 1D clipped method as the 2D Product mapping on a 1 x 6 grid.

    alpha = beta = 3 makes the index a clip at 3; the row index is always 0 (row bucket
    H = 3 of S = 7).  The Shaw page indexes its table by j - i; the bucket here uses the
    query-minus-key offset, so the page's table enters mirrored.
    """
    spec = Spec(1, 6, mode="contextual", terms={"k", "v"}, map="piecewise",
                alpha=3.0, beta=3.0, gamma=10.0)
    _, s, nb = num_buckets(spec)
    rk = np.zeros((1, nb, 4))
    rv = np.zeros((1, nb, 4))
    for c in range(7):
        src = 6 - c if mirror else c
        rk[0, 3 * s + c] = a_k[src]
        rv[0, 3 * s + c] = a_v[src]
    return spec, rk, rv


def test_shaw_page_printed_weights(golden_dir):
    # Shaw-style page, "Testing the Implementation": printed 6x6 weights (3 decimals).
    printed = np.loadtxt(os.path.join(golden_dir, "shaw_1d_weights.txt"))
    q, k, v, a_k, a_v = _shaw_page_setup()
    spec, rk, rv = _shaw_as_2d(a_k, a_v)
    o, _, wts = attention(spec, q[None, None], k[None, None], v[None, None], rk=rk, rv=rv,
                          return_weights=True)
    err = np.abs(wts[(0, 0, 0)] - printed).max()
    assert err <= 5e-4 + 1e-12, err
    # discrimination: the unmirrored table (wrong offset sign) and no table both miss
    spec, rk2, rv2 = _shaw_as_2d(a_k, a_v, mirror=False)
    _, _, w2 = attention(spec, q[None, None], k[None, None], v[None, None], rk=rk2, rv=rv2,
                         return_weights=True)
    assert np.abs(w2[(0, 0, 0)] - printed).max() > 0.1
    _, _, w3 = attention(spec, q[None, None], k[None, None], v[None, None],
                         rk=np.zeros_like(rk), rv=np.zeros_like(rv), return_weights=True)
    assert np.abs(w3[(0, 0, 0)] - printed).max() > 0.1
    # the value term of the page's layer, written independently: sum_j a_ij (v_j + a^V[j-i])
    a = wts[(0, 0, 0)]
    ref = np.zeros((6, 4))
    for i in range(6):
        for j in range(6):
            ref[i] += a[i, j] * (v[j] + a_v[max(-3, min(3, j - i)) + 3])
    np.testing.assert_allclose(o[0, 0], ref, atol=1e-12)


def test_windows_equal_prepartitioned_batch():
    # Attention inside non-overlapping windows of a grid equals attention over a batch of
    # the windows cut out beforehand (Swin relative-bias record, Conditions).
    G, M, d = 6, 3, 4
    spec = Spec(G, G, window=M, mode="bias", map="swin", tables_per_head=True)
    rng = np.random.default_rng(4)
    q, k, v, tabs = _inputs(spec, 2, 2, d, rng, per_head=True)
    o, lse = attention(spec, q, k, v, **tabs)
    wspec = Spec(M, M, window=0, mode="bias", map="swin", tables_per_head=True)
    for u in range(spec.units_per_image):
        idx = unit_token_indices(spec, u)
        o2, l2 = attention(wspec, q[:, :, idx], k[:, :, idx], v[:, :, idx], **tabs)
        np.testing.assert_allclose(o[:, :, idx], o2, atol=1e-13)
        np.testing.assert_allclose(lse[:, :, idx], l2, atol=1e-13)


def test_efficient_form_identity():
    # iRPE page, Method, eqs. 26-28: q_i . r_b computed once per bucket and gathered equals
    # the per-pair product; the value term equals per-bucket weight sums times r^V.
    spec = Spec(5, 5, prefix=1, mode="contextual", terms={"k", "q", "v"}, map="piecewise",
                alpha=1.9, beta=3.8, gamma=15.2)
    rng = np.random.default_rng(8)
    d = 8
    q, k, v, tabs = _inputs(spec, 1, 1, d, rng)
    o, lse, wts = attention(spec, q, k, v, return_weights=True, **tabs)
    bm = bucket_map_array(spec)
    has = bm >= 0
    Q, K, V = q[0, 0], k[0, 0], v[0, 0]
    tk = Q @ tabs["rk"][0].T           # [T, buckets]
    tq = K @ tabs["rq"][0].T
    T = Q.shape[0]
    rows = np.arange(T)[:, None]
    cols = np.arange(T)[None, :]
    lg = (Q @ K.T + np.where(has, tk[rows, np.where(has, bm, 0)], 0)
          + np.where(has, tq[cols, np.where(has, bm, 0)], 0)) / math.sqrt(d)
    a = torch.softmax(torch.from_numpy(lg), -1).numpy()
    np.testing.assert_allclose(wts[(0, 0, 0)], a, atol=1e-13)
    _, _, nb = num_buckets(spec)
    W = np.zeros((T, nb))
    for i in range(T):
        for j in range(T):
            if has[i, j]:
                W[i, bm[i, j]] += a[i, j]
    np.testing.assert_allclose(o[0, 0], a @ V + W @ tabs["rv"][0], atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], torch.logsumexp(torch.from_numpy(lg), -1).numpy(),
                               atol=1e-13)


def test_scale_placement():
    # Contextual terms sit inside the scale (iRPE page, DeiT steps, step 3); the Swin bias
    # is added after it (Swin relative-bias record, "The claim").  Doubling s with a zero
    # table must equal the plain attention at 2s; a bias table is not scaled by s.
    rng = np.random.default_rng(12)
    d = 4
    spec_b = Spec(3, 3, window=3, mode="bias", map="swin", scale=0.25)
    q, k, v, tabs = _inputs(spec_b, 1, 1, d, rng)
    _, _, w = attention(spec_b, q, k, v, return_weights=True, **tabs)
    bm = bucket_map_array(spec_b)
    lg = q[0, 0] @ k[0, 0].T * 0.25 + tabs["bias"][0][bm]
    np.testing.assert_allclose(w[(0, 0, 0)], torch.softmax(torch.from_numpy(lg), -1).numpy(),
                               atol=1e-13)
    spec_c = Spec(3, 3, mode="contextual", terms={"k"}, map="piecewise", alpha=1.0, beta=2.0,
                  gamma=4.0, scale=0.25)
    _, _, nb = num_buckets(spec_c)
    rk = rng.standard_normal((1, nb, d))
    _, _, w = attention(spec_c, q, k, v, rk=rk, return_weights=True)
    bm = bucket_map_array(spec_c)
    lg = (q[0, 0] @ k[0, 0].T + np.einsum("id,ijd->ij", q[0, 0], rk[0][bm])) * 0.25
    np.testing.assert_allclose(w[(0, 0, 0)], torch.softmax(torch.from_numpy(lg), -1).numpy(),
                               atol=1e-13)


# ------------------------------------------------------------------ Cross mapping

def _shaw_as_cross(a_k, a_v, axis):
    """The 1D clipped method as the Cross mapping on a 1 x 6 (axis "x") or 6 x 1
    (axis "y") grid: the moving axis's half of each table holds the page's table
    (mirrored, as in _shaw_as_2d), the other half is zero."""
    gh, gw = (1, 6) if axis == "x" else (6, 1)
    spec = Spec(gh, gw, mode="contextual", terms={"k", "v"}, map="piecewise",
                alpha=3.0, beta=3.0, gamma=10.0, method="cross")
    _, s, nb = num_buckets(spec)
    assert nb == 2 * s == 14
    rk = np.zeros((1, nb, 4))
    rv = np.zeros((1, nb, 4))
    base = s if axis == "x" else 0
    for c in range(7):
        rk[0, base + c] = a_k[6 - c]
        rv[0, base + c] = a_v[6 - c]
    return spec, rk, rv


@pytest.mark.parametrize("axis", ["x", "y"])
def test_cross_shaw_page_printed_weights(golden_dir, axis):
    # iRPE page, Method, Cross (eqs. 22-24): on a grid with one row (one column) the
    # row-offset (column-offset) index is always 0, so with that half of the table at
    # zero the method is the 1D clipped encoding of the Shaw-style page, whose printed
    # 6x6 weights (3 decimals) it must reproduce.  Pins the split of the table into a
    # row half [0, S) and a column half [S, 2S).
    printed = np.loadtxt(os.path.join(golden_dir, "shaw_1d_weights.txt"))
    q, k, v, a_k, a_v = _shaw_page_setup()
    spec, rk, rv = _shaw_as_cross(a_k, a_v, axis)
    o, _, wts = attention(spec, q[None, None], k[None, None], v[None, None], rk=rk, rv=rv,
                          return_weights=True)
    assert np.abs(wts[(0, 0, 0)] - printed).max() <= 5e-4 + 1e-12
    a = wts[(0, 0, 0)]
    ref = np.zeros((6, 4))
    for i in range(6):
        for j in range(6):
            ref[i] += a[i, j] * (v[j] + a_v[max(-3, min(3, j - i)) + 3])
    np.testing.assert_allclose(o[0, 0], ref, atol=1e-12)
    # the same table in the other half misses (its axis never moves: a constant term)
    other = "y" if axis == "x" else "x"
    _, rk2, rv2 = _shaw_as_cross(a_k, a_v, other)
    _, _, w2 = attention(spec, q[None, None], k[None, None], v[None, None], rk=rk2, rv=rv2,
                         return_weights=True)
    assert np.abs(w2[(0, 0, 0)] - printed).max() > 0.1


CROSS_TINY = [
    Spec(3, 4, prefix=1, mode="contextual", terms={"k", "q", "v"}, map="piecewise",
         alpha=0.9, beta=1.7, gamma=3.0, method="cross"),
    Spec(4, 4, window=2, mode="bias", map="swin", method="cross"),
    Spec(3, 5, prefix=1, mode="bias", map="piecewise", alpha=1.0, beta=2.0, gamma=4.0, method="cross"),
]


@pytest.mark.parametrize("spec", CROSS_TINY)
def test_cross_literal_matches_vectorised(spec):
    rng = np.random.default_rng(17)
    q, k, v, tabs = _inputs(spec, 2, 2, 5, rng, per_head=True)
    o1, l1 = attention_literal(spec, q, k, v, **tabs)
    o2, l2 = attention(spec, q, k, v, **tabs)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)


@pytest.mark.parametrize("spec", CROSS_TINY)
def test_cross_is_product_of_summed_rows(spec):
    # The two encodings of a Cross pair add (eqs. 22-24), so a Cross table T equals the
    # Product table P[by * S + bx] = T[by] + T[S + bx] over the same index function.
    rng = np.random.default_rng(19)
    q, k, v, tabs = _inputs(spec, 2, 2, 5, rng, per_head=True)
    _, s, _ = num_buckets(spec)
    prod = Spec(**{f: getattr(spec, f) for f in spec.__dataclass_fields__ if f != "method"})
    ptabs = {}
    for n, t in tabs.items():
        by = np.arange(s * s) // s
        bx = s + np.arange(s * s) % s
        ptabs[n] = t[:, by] + t[:, bx]
    o1, l1 = attention(spec, q, k, v, **tabs)
    o2, l2 = attention(prod, q, k, v, **ptabs)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)
    # dropping either half changes the result
    for half in (slice(0, s), slice(s, 2 * s)):
        t2 = {n: t.copy() for n, t in tabs.items()}
        for t in t2.values():
            t[:, half] = 0.0
        o3, _ = attention(spec, q, k, v, **t2)
        assert np.abs(o3 - o1).max() > 1e-3
