"""Seeded random attention configurations shared by the GPU parity tests of the
forward and the backward (shapes and parameters only; no arithmetic of the
method)."""

import numpy as np

from oracle import Spec, num_buckets
from vision_transformer_attention_amd.workloads import WORKLOADS


def random_config(i):
    """A seeded configuration: unit widths 1..160 (a third over 64 columns), every
    mode, map, method, dtype and head dim; shapes kept to what one CU's LDS plan
    holds (Swin-map tables grow as (2 max(R, C) - 1)^2) and the oracle finishes
    in well under a second."""
    rng = np.random.default_rng(12000 + i)
    pick = lambda xs: xs[int(rng.integers(len(xs)))]
    dtype = pick(["bf16", "bf16", "fp32"])
    d = pick([16, 32, 64])
    mode = pick(["none", "bias", "contextual", "contextual"])
    terms = frozenset()
    if mode == "contextual":
        terms = frozenset(t for t in "kqv" if rng.random() < 0.6) or frozenset("k")
    window = 0
    if rng.random() < 0.25:
        window = int(rng.integers(2, 9))
        gh, gw = window * int(rng.integers(1, 3)), window * int(rng.integers(1, 4))
        prefix = 0
    else:
        gw = int(rng.integers(65, 161)) if rng.random() < 1 / 3 else int(rng.integers(1, 40))
        gh = int(rng.integers(1, max(2, min(9, 600 // gw + 1))))
        prefix = pick([0, 0, 1, 2])
    unit = max(window or gh, window or gw)
    maps = ["piecewise", "piecewise"]
    if mode != "none" and unit <= (16 if mode == "bias" else 8):
        maps.append("swin")
    if mode != "none":
        maps += ["euclidean", "quantized"]
    m = pick(maps) if mode != "none" else "swin"
    method = "cross" if (mode != "none" and m in ("piecewise", "swin") and rng.random() < 0.25) else "product"
    a = float(rng.uniform(0.8, 3.0))
    b = a + float(rng.uniform(0.5, 4.0))
    g = b + float(rng.uniform(1.0, 20.0))
    w = WORKLOADS["deit_s_irpe_k"].resized(batch=int(rng.integers(1, 3)), heads=int(rng.integers(1, 4)), head_dim=d, grid_h=gh, grid_w=gw,
                   window=window, prefix=prefix, mode=mode, terms=terms, map=m, alpha=a, beta=b, gamma=g,
                   reading=pick(["capped", "trunc"]), dtype=dtype, tables_per_head=bool(rng.random() < 0.4),
                   method=method)
    if mode == "none":
        return w
    spec = Spec(w.grid_h, w.grid_w, window=w.window, prefix=w.prefix, mode=w.mode, terms=w.terms, map=w.map,
                alpha=w.alpha, beta=w.beta, gamma=w.gamma, reading=w.reading, tables_per_head=w.tables_per_head,
                method=w.method)
    return w.resized(table_rows=num_buckets(spec)[2])
