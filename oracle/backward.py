"""Backward pass of the attention forward (oracle, fp64).

Test infrastructure only (see the package docstring).

Gradients of o = attention(q, k, v, tables) (``oracle.attention``) with respect
to every input, given the gradient dO of the output, written from the
definition (iRPE page, Method, eqs. 13-17; Swin relative-bias record, "The
claim").  Per unit and (batch, head), with s the logit scale, P the softmax
weights and b(i, j) the table rows of a pair (none for prefix pairs; two for
the Cross mapping):

    dP_ij  = dO_i . (v_j + [V] rV[b])
    dL_ij  = P_ij (dP_ij - sum_j' P_ij' dP_ij')          (softmax)
    dq_i   = s sum_j dL_ij (k_j + [K] rK[b])
    dk_j   = s sum_i dL_ij (q_i + [Q] rQ[b])
    dv_j   = sum_i P_ij dO_i
    drK[b] += s dL_ij q_i,  drQ[b] += s dL_ij k_j,  drV[b] += P_ij dO_i,  dB[b] += dL_ij

Contextual terms sit inside the scale (logit = (q.k + rho) s); the bias is
added after it (logit = q.k s + B).  Shared tables sum over heads.
Parity pins: central finite differences of the forward oracle (tests).
"""

import math

import numpy as np

from .attention import _check_tables, _head_table, pair_rows_arrays, unit_token_indices


def attention_backward(spec, q, k, v, do, bias=None, rk=None, rq=None, rv=None):
    """Returns a dict of float64 gradients: dq, dk, dv ([B, H, N, d]) and, for the
    tables present, dbias / drk / drq / drv shaped like the tables."""
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    B, H, N, d = q.shape
    bias_t, rk_t, rq_t, rv_t = _check_tables(spec, H, d, bias, rk, rq, rv)
    s = spec.scale if spec.scale is not None else 1.0 / math.sqrt(d)
    out = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v)}
    grads = {}
    for name, t in (("dbias", bias_t), ("drk", rk_t), ("drq", rq_t), ("drv", rv_t)):
        if t is not None:
            grads[name] = np.zeros_like(t)

    def tidx(t, h):
        return h if t.shape[0] > 1 else 0

    for u in range(spec.units_per_image):
        idx = np.array(unit_token_indices(spec, u), dtype=np.int64)
        rows = pair_rows_arrays(spec, u)
        has = rows[0] >= 0
        safes = [np.where(has, r, 0) for r in rows]
        for b in range(B):
            for h in range(H):
                Q, K, V, dO = q[b, h, idx], k[b, h, idx], v[b, h, idx], do[b, h, idx]
                T = len(idx)
                # forward quantities
                logits = Q @ K.T
                if spec.mode == "contextual":
                    for sf in safes:
                        if rk_t is not None:
                            logits += np.where(has, np.einsum("id,ijd->ij", Q, _head_table(rk_t, h)[sf]), 0.0)
                        if rq_t is not None:
                            logits += np.where(has, np.einsum("jd,ijd->ij", K, _head_table(rq_t, h)[sf]), 0.0)
                    logits = logits * s
                elif spec.mode == "bias":
                    logits = logits * s
                    for sf in safes:
                        logits += np.where(has, _head_table(bias_t, h)[sf], 0.0)
                else:
                    logits = logits * s
                mx = logits.max(axis=1, keepdims=True)
                e = np.exp(logits - mx)
                P = e / e.sum(axis=1, keepdims=True)
                # backward
                dP = dO @ V.T
                if rv_t is not None:
                    for sf in safes:
                        dP += np.where(has, np.einsum("id,ijd->ij", dO, _head_table(rv_t, h)[sf]), 0.0)
                dL = P * (dP - (P * dP).sum(axis=1, keepdims=True))
                dlog = dL * s          # the scale multiplies q.k and the contextual terms
                dq = dlog @ K
                dk = dlog.T @ Q
                dv = P.T @ dO
                if spec.mode == "contextual":
                    for sf in safes:
                        m = has[:, :, None]
                        if rk_t is not None:
                            tab = _head_table(rk_t, h)[sf]                     # [i, j, d]
                            dq += np.einsum("ij,ijd->id", dlog, tab * m)
                            g = grads["drk"][tidx(rk_t, h)]
                            np.add.at(g, sf[has], (dlog[:, :, None] * Q[:, None, :])[has])
                        if rq_t is not None:
                            tab = _head_table(rq_t, h)[sf]
                            dk += np.einsum("ij,ijd->jd", dlog, tab * m)
                            g = grads["drq"][tidx(rq_t, h)]
                            np.add.at(g, sf[has], (dlog[:, :, None] * K[None, :, :])[has])
                        if rv_t is not None:
                            g = grads["drv"][tidx(rv_t, h)]
                            np.add.at(g, sf[has], (P[:, :, None] * dO[:, None, :])[has])
                elif spec.mode == "bias":
                    for sf in safes:
                        g = grads["dbias"][tidx(bias_t, h)]
                        np.add.at(g, sf[has], dL[has])
                out["dq"][b, h, idx] += dq
                out["dk"][b, h, idx] += dk
                out["dv"][b, h, idx] += dv
    out.update(grads)
    return out
