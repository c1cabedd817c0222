"""Attention forward with 2D relative position terms (oracle, fp64).

Test infrastructure only (see the package docstring).

Per unit (one window, or one whole grid), per batch b and head h, for query
token i and key token j of the unit (prefix tokens first):

    c_ij   = q_i . k_j                                   (iRPE page, eqs. 1-3)
    b_ij   = bucket id of the pair, -1 if i or j is a prefix token
    rho_ij = [K] q_i . rK[b_ij] + [Q] k_j . rQ[b_ij]     (eqs. 13, 15, 16)

With the Cross mapping (eqs. 22-24) a pair has two table rows, a row-offset
row and a column-offset row, and every table term above is the sum of the
two rows' terms (X[b_ij] reads X[by_ij] + X[bx_ij]).
    logit  = (c_ij + rho_ij) * s             contextual mode (eq. 13; the
                                             position term is added before the
                                             division by sqrt(d), Method,
                                             "Applying iRPE to a DeiT-style
                                             model", step 3)
           = c_ij * s + B[b_ij]              bias mode (Swin relative-bias
                                             record, "The claim":
                                             SoftMax(QK^T/sqrt(d) + B) V)
    a_ij   = softmax over all j of the unit (prefix included)
    o_i    = sum_j a_ij (v_j + [V] rV[b_ij])            (eq. 17, value term
                                             weighted by the attention)
    lse_i  = log sum_j exp(logit_ij)

A term whose bucket is -1 contributes 0.  s defaults to 1/sqrt(d).

Tables: bias [heads or 1][S*S]; rK, rQ, rV [heads or 1][S*S][d]; a leading
size of 1 (or ``spec.tables_per_head`` False) means one table shared by all
heads (iRPE page, Method, "Other design choices").

Tensor layout: q, k, v and the output are [B, H, N, d] with N = prefix +
grid_h * grid_w tokens, grid tokens in row-major order.
"""

import math

import numpy as np

from .buckets import num_buckets, pair_rows, unit_positions


def unit_token_indices(spec, unit):
    """Token indices of one unit, in unit order (prefix first)."""
    return [t for t, _ in unit_positions(spec, unit)]


def _axis_table(spec, length):
    """g(x) for x in [-(length-1), length-1] via the scalar definition."""
    return np.array([spec.g(x) for x in range(-(length - 1), length)], dtype=np.int64)


def bucket_map_array(spec, unit=0):
    """Bucket ids of one unit as an int64 [T, T] array (vectorised form).

    Same definition as ``buckets.pair_bucket`` (per-pair offset -> per-axis
    index -> row-major id), evaluated for all pairs at once; the tests check
    the two agree.
    """
    toks = unit_positions(spec, unit)
    h, s, _ = num_buckets(spec)
    n_pre = spec.prefix
    ys = np.array([p[0] for _, p in toks[n_pre:]], dtype=np.int64)
    xs = np.array([p[1] for _, p in toks[n_pre:]], dtype=np.int64)
    t = len(toks)
    out = np.full((t, t), -1, dtype=np.int64)
    if len(ys) == 0:
        return out
    span_y = int(ys.max() - ys.min()) + 1
    span_x = int(xs.max() - xs.min()) + 1
    gy_tab = _axis_table(spec, span_y)
    gx_tab = _axis_table(spec, span_x)
    if np.abs(gy_tab).max() > h or np.abs(gx_tab).max() > h:
        raise ValueError("index outside the table half-width")
    dy = ys[:, None] - ys[None, :]
    dx = xs[:, None] - xs[None, :]
    gy = gy_tab[dy + (span_y - 1)]
    gx = gx_tab[dx + (span_x - 1)]
    out[n_pre:, n_pre:] = (gy + h) * s + (gx + h)
    return out


def pair_rows_arrays(spec, unit=0):
    """Table rows of every pair of one unit: a list of int64 [T, T] arrays
    (-1 where the pair has no position term) whose rows' encodings add up:
    the Product id alone, or the Cross mapping's row-offset and
    column-offset rows (same definition as ``buckets.pair_rows``)."""
    if spec.undirected:
        toks = unit_positions(spec, unit)
        h, _, _ = num_buckets(spec)
        cache = {}
        out = np.full((len(toks), len(toks)), -1, dtype=np.int64)
        for i, (_, pi) in enumerate(toks):
            for j, (_, pj) in enumerate(toks):
                if pi is None or pj is None:
                    continue
                key = (abs(pi[0] - pj[0]), abs(pi[1] - pj[1]))
                if key not in cache:
                    cache[key] = spec.u(*key) + h
                out[i, j] = cache[key]
        return [out]
    if spec.method != "cross":
        return [bucket_map_array(spec, unit)]
    h, s, _ = num_buckets(spec)
    prod = bucket_map_array(spec, unit)
    has = prod >= 0
    gy = np.where(has, prod // s, -1)          # g(dy) + H
    gx = np.where(has, s + prod % s, -1)       # S + g(dx) + H
    return [gy, gx]


def _check_tables(spec, heads, d, bias, rk, rq, rv):
    _, _, nb = num_buckets(spec)

    def chk(name, t, want_d):
        if t is None:
            return None
        t = np.asarray(t, dtype=np.float64)
        if want_d:
            if t.ndim == 2:
                t = t[None]
            if t.shape[1:] != (nb, d):
                raise ValueError(f"{name} must be [heads|1][{nb}][{d}], got {t.shape}")
        else:
            if t.ndim == 1:
                t = t[None]
            if t.shape[1:] != (nb,):
                raise ValueError(f"{name} must be [heads|1][{nb}], got {t.shape}")
        if t.shape[0] not in (1, heads):
            raise ValueError(f"{name} leading size must be 1 or {heads}")
        return t

    if spec.mode == "bias" and bias is None:
        raise ValueError("bias mode needs a bias table")
    if spec.mode == "contextual":
        for term, t in (("k", rk), ("q", rq), ("v", rv)):
            if term in spec.terms and t is None:
                raise ValueError(f"contextual term {term} needs its table")
    return (chk("bias", bias, False) if spec.mode == "bias" else None,
            chk("rk", rk, True) if "k" in spec.terms and spec.mode == "contextual" else None,
            chk("rq", rq, True) if "q" in spec.terms and spec.mode == "contextual" else None,
            chk("rv", rv, True) if "v" in spec.terms and spec.mode == "contextual" else None)


def _head_table(t, h):
    if t is None:
        return None
    return t[h] if t.shape[0] > 1 else t[0]


def attention(spec, q, k, v, bias=None, rk=None, rq=None, rv=None,
              return_weights=False, units=None, heads_sel=None, batch_sel=None):
    """Vectorised oracle.  q, k, v: [B, H, N, d] (any float dtype; upcast).

    Returns (o, lse) as float64 arrays [B, H, N, d] and [B, H, N]; with
    ``return_weights`` also a dict {(b, h, unit): a [T, T]}.
    ``units``/``heads_sel``/``batch_sel`` restrict the work to a subset (the
    untouched outputs stay NaN); used to time or check a bounded sample.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    if N != spec.tokens_per_image:
        raise ValueError(f"N = {N}, spec expects {spec.tokens_per_image}")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one shape")
    bias_t, rk_t, rq_t, rv_t = _check_tables(spec, H, d, bias, rk, rq, rv)
    s = spec.scale if spec.scale is not None else 1.0 / math.sqrt(d)

    o = np.full((B, H, N, d), np.nan)
    lse = np.full((B, H, N), np.nan)
    weights = {}
    unit_list = range(spec.units_per_image) if units is None else units
    b_list = range(B) if batch_sel is None else batch_sel
    h_list = range(H) if heads_sel is None else heads_sel

    for u in unit_list:
        idx = np.array(unit_token_indices(spec, u), dtype=np.int64)
        rows = pair_rows_arrays(spec, u)
        has = rows[0] >= 0
        safes = [np.where(has, r, 0) for r in rows]
        T = len(idx)
        chunk = max(1, (1 << 25) // max(1, T * d))
        for b in b_list:
            for h in h_list:
                Q, K, V = q[b, h, idx], k[b, h, idx], v[b, h, idx]
                logits = np.empty((T, T))
                out_v = np.zeros((T, d))
                for i0 in range(0, T, chunk):
                    i1 = min(T, i0 + chunk)
                    c = Q[i0:i1] @ K.T
                    m = has[i0:i1]
                    if spec.mode == "contextual":
                        rho = np.zeros_like(c)
                        for safe in safes:
                            bid = safe[i0:i1]
                            if rk_t is not None:
                                tab = _head_table(rk_t, h)[bid]            # [i, j, d]
                                rho += np.where(m, np.einsum("id,ijd->ij", Q[i0:i1], tab), 0.0)
                            if rq_t is not None:
                                tab = _head_table(rq_t, h)[bid]
                                rho += np.where(m, np.einsum("jd,ijd->ij", K, tab), 0.0)
                        logits[i0:i1] = (c + rho) * s
                    elif spec.mode == "bias":
                        add = np.zeros_like(c)
                        for safe in safes:
                            add += np.where(m, _head_table(bias_t, h)[safe[i0:i1]], 0.0)
                        logits[i0:i1] = c * s + add
                    else:
                        logits[i0:i1] = c * s
                mx = logits.max(axis=1, keepdims=True)
                e = np.exp(logits - mx)
                den = e.sum(axis=1, keepdims=True)
                a = e / den
                out = a @ V
                if rv_t is not None:
                    tv = _head_table(rv_t, h)
                    for i0 in range(0, T, chunk):
                        i1 = min(T, i0 + chunk)
                        for safe in safes:
                            tab = tv[safe[i0:i1]] * has[i0:i1, :, None]
                            out_v[i0:i1] += np.einsum("ij,ijd->id", a[i0:i1], tab)
                    out = out + out_v
                o[b, h, idx] = out
                lse[b, h, idx] = (mx + np.log(den))[:, 0]
                if return_weights:
                    weights[(b, h, u)] = a
    if return_weights:
        return o, lse, weights
    return o, lse


def attention_literal(spec, q, k, v, bias=None, rk=None, rq=None, rv=None):
    """Pure-Python loop oracle for tiny shapes: one pair at a time.

    Follows the same definition as ``attention`` with no vectorisation and
    no library calls beyond math.exp/log; used to cross-check ``attention``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    bias_t, rk_t, rq_t, rv_t = _check_tables(spec, H, d, bias, rk, rq, rv)
    s = spec.scale if spec.scale is not None else 1.0 / math.sqrt(d)
    o = np.full((B, H, N, d), np.nan)
    lse = np.full((B, H, N), np.nan)
    for u in range(spec.units_per_image):
        toks = unit_positions(spec, u)
        for b in range(B):
            for h in range(H):
                for ti, pi in toks:
                    logits = []
                    for tj, pj in toks:
                        c = sum(q[b, h, ti, e] * k[b, h, tj, e] for e in range(d))
                        rows = pair_rows(spec, pi, pj)
                        if spec.mode == "contextual":
                            rho = 0.0
                            for bid in rows:
                                if rk_t is not None:
                                    row = _head_table(rk_t, h)[bid]
                                    rho += sum(q[b, h, ti, e] * row[e] for e in range(d))
                                if rq_t is not None:
                                    row = _head_table(rq_t, h)[bid]
                                    rho += sum(k[b, h, tj, e] * row[e] for e in range(d))
                            logits.append((c + rho) * s)
                        elif spec.mode == "bias":
                            add = sum(_head_table(bias_t, h)[bid] for bid in rows)
                            logits.append(c * s + add)
                        else:
                            logits.append(c * s)
                    mx = max(logits)
                    ex = [math.exp(x - mx) for x in logits]
                    den = sum(ex)
                    acc = [0.0] * d
                    for (tj, pj), w in zip(toks, ex):
                        a = w / den
                        rows = pair_rows(spec, pi, pj)
                        for e in range(d):
                            val = v[b, h, tj, e]
                            if rv_t is not None:
                                for bid in rows:
                                    val += _head_table(rv_t, h)[bid][e]
                            acc[e] += a * val
                    o[b, h, ti] = acc
                    lse[b, h, ti] = mx + math.log(den)
    return o, lse
