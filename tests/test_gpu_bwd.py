"""GPU parity of the backward pass (rpe_attn_bwd, through the C ABI) against the
fp64 oracle backward.  The log-sum-exp comes from the GPU forward, as it would in
use; gradients are float32.  Tolerances, relative to the largest reference
gradient of each tensor: 2e-4 for fp32 inputs (float32 sums over at most a few
hundred terms), 2e-2 for bf16 inputs (the forward's log-sum-exp sums bf16-rounded
weights, which shifts the recomputed weights by up to ~2^-8 relative)."""

import numpy as np
import pytest

from oracle import Spec, num_buckets
from oracle.backward import attention_backward
from vision_transformer_attention_amd.workloads import WORKLOADS, make_inputs, round_to_dtype
from random_configs import random_config

pytestmark = pytest.mark.gpu

REL = {"bf16": 2e-2, "fp32": 2e-4}


@pytest.fixture(scope="module")
def dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vision_transformer_attention_amd as pkg
    pkg.load()
    return torch.device("cuda:0")


def _spec(w):
    return Spec(w.grid_h, w.grid_w, window=w.window, prefix=w.prefix, mode=w.mode, terms=w.terms, map=w.map,
                alpha=w.alpha, beta=w.beta, gamma=w.gamma, reading=w.reading, tables_per_head=w.tables_per_head,
                method=w.method)


def _fit(w):
    return w.resized(table_rows=num_buckets(_spec(w))[2]) if w.mode != "none" else w


_D = WORKLOADS["deit_s_irpe_k"]
_S = WORKLOADS["swin_t_w7"]
CASES = [
    ("bias, 7x7 windows, per head, bf16", _S.resized(batch=2, heads=3, grid_h=14, grid_w=14)),
    ("iRPE bias, global 14x14 + cls, bf16", _D.resized(batch=1, heads=2, mode="bias", terms=frozenset(),
                                                        tables_per_head=True)),
    ("contextual K, global 14x14 + cls, bf16", _D.resized(batch=1, heads=2)),
    ("contextual KQV, 6x7 + cls, fp32", _D.resized(batch=2, heads=2, grid_h=6, grid_w=7, terms=frozenset("kqv"),
                                                   dtype="fp32")),
    ("contextual QV, 4x4 windows, per head, fp32 d16", _D.resized(batch=1, heads=2, head_dim=16, grid_h=8, grid_w=8,
                                                                   window=4, prefix=0, terms=frozenset("qv"),
                                                                   dtype="fp32", tables_per_head=True)),
    ("contextual KQV, 5x9 + cls, bf16 d32", _D.resized(batch=1, heads=2, head_dim=32, grid_h=5, grid_w=9,
                                                       terms=frozenset("kqv"))),
    ("no position terms, 9x9 + cls, fp32", _D.resized(batch=1, heads=2, grid_h=9, grid_w=9, mode="none",
                                                      terms=frozenset(), map="swin", dtype="fp32")),
    # bf16 with head dim 16: the per-element kernels
    ("contextual KQV, 6x7 + cls, bf16 d16", _D.resized(batch=2, heads=2, head_dim=16, grid_h=6, grid_w=7,
                                                       terms=frozenset("kqv"))),
    # the matrix-core kernels on windowed units with per-head tables
    ("contextual KQV, 7x7 windows, per head, bf16 d32", _D.resized(batch=2, heads=2, head_dim=32, grid_h=14,
                                                                   grid_w=14, window=7, prefix=0,
                                                                   terms=frozenset("kqv"), tables_per_head=True)),
    ("contextual K, 9x9 + 2 prefix, per head, bf16 d64", _D.resized(batch=1, heads=3, grid_h=9, grid_w=9, prefix=2,
                                                                    tables_per_head=True)),
    # 47 x 47 = 2209 table entries: the row pass sums into global memory (more than its LDS takes)
    ("bias, one 24x24 window, fp32 d16", _S.resized(batch=1, heads=1, head_dim=16, grid_h=24, grid_w=24,
                                                     window=24, dtype="fp32")),
    # 289 buckets with the query term: the key-column bucket sums take the global-memory
    # kernel (more than 256 buckets), in fp32 and on the bf16 matrix-core path
    ("contextual Q, 289 buckets, 9x9 + cls, fp32 d16", _D.resized(batch=1, heads=2, head_dim=16, grid_h=9,
                                                                   grid_w=9, terms=frozenset("q"), alpha=3.8,
                                                                   beta=7.6, gamma=30.4, dtype="fp32")),
    ("contextual Q, 289 buckets, 9x9 + cls, bf16 d64", _D.resized(batch=1, heads=2, grid_h=9, grid_w=9,
                                                                   terms=frozenset("q"), alpha=3.8, beta=7.6,
                                                                   gamma=30.4)),
    # Cross mapping (2S-row tables, each pair reads a row-offset and a column-offset row)
    ("cross contextual K, global 14x14 + cls, bf16", _D.resized(batch=1, heads=2, method="cross")),
    ("cross bias, 7x7 windows, per head, bf16", _S.resized(batch=2, heads=3, grid_h=14, grid_w=14,
                                                            method="cross")),
    ("cross contextual KQV, 4x4 windows, fp32 d16", _D.resized(batch=2, heads=2, head_dim=16, grid_h=8,
                                                                grid_w=8, window=4, prefix=0,
                                                                terms=frozenset("kqv"), dtype="fp32",
                                                                method="cross")),
    ("cross contextual QV, 9x13, per head, bf16 d32", _D.resized(batch=1, heads=3, head_dim=32, grid_h=9,
                                                                  grid_w=13, prefix=0, terms=frozenset("qv"),
                                                                  tables_per_head=True, method="cross")),
    ("cross contextual KQV, 6x7 + cls, bf16 d16", _D.resized(batch=2, heads=2, head_dim=16, grid_h=6, grid_w=7,
                                                             terms=frozenset("kqv"), method="cross")),
    # undirected maps (S-row tables, rows u + H; rows below H are read by no pair)
    ("euclidean bias, 14x14 + cls, per head, bf16", _D.resized(batch=1, heads=2, mode="bias",
                                                               terms=frozenset(), map="euclidean",
                                                               tables_per_head=True)),
    # (the forward runs an undirected map on its expansion over raw offsets: 11 x 11 rows here)
    ("quantized contextual KV, 5x6 + cls, fp32", _D.resized(batch=2, heads=2, grid_h=5, grid_w=6,
                                                            terms=frozenset("kv"), map="quantized",
                                                            dtype="fp32")),
    ("euclidean (rounded) contextual KQV, 7x7 windows, bf16 d32",
     _D.resized(batch=1, heads=2, head_dim=32, grid_h=14, grid_w=14, window=7, prefix=0, terms=frozenset("kqv"),
                map="euclidean_rounded")),
    ("quantized (squared) contextual K, 14x14 + cls, bf16", _D.resized(batch=1, heads=2,
                                                                      map="quantized_squared")),
    # rows wider than 64 columns (the forward's log-sum-exp from its 128-slot rows)
    ("contextual KQV, 3x100 + cls, bf16 d32", _D.resized(batch=1, heads=2, head_dim=32, grid_h=3, grid_w=100,
                                                         terms=frozenset("kqv"))),
    ("bias, 2x130, per head, fp32 d16", _D.resized(batch=1, heads=2, head_dim=16, grid_h=2, grid_w=130, prefix=0,
                                                    mode="bias", terms=frozenset(), tables_per_head=True,
                                                    dtype="fp32")),
]


@pytest.mark.parametrize("label,w", CASES)
def test_backward_parity(dev, label, w):
    w = _fit(w)
    print("[case] backward", label, w.qkv_shape, flush=True)
    _check_backward(dev, w, 9950)


def _random_backward_configs(n):
    """The first n seeded random configurations the backward takes (undirected
    maps: (R-1)^2 + (C-1)^2 < 16384 for a unit of R x C positions)."""
    out, k = [], 100
    while len(out) < n:
        w = random_config(k)
        r, c = (w.window, w.window) if w.window else (w.grid_h, w.grid_w)
        if not (w.map in ("euclidean", "euclidean_rounded", "quantized", "quantized_squared")
                and (r - 1) ** 2 + (c - 1) ** 2 >= 16384):
            out.append((k, w))
        k += 1
    return out


@pytest.mark.parametrize("k,w", _random_backward_configs(12))
def test_backward_random_configs(dev, k, w):
    print("[case] backward random config", k, w.qkv_shape, w.mode, "".join(sorted(w.terms)), w.map, w.method,
          w.dtype, "grid", (w.grid_h, w.grid_w), "window", w.window, "prefix", w.prefix, flush=True)
    _check_backward(dev, w, 12700 + k)


def _check_backward(dev, w, seed):
    import torch
    import vision_transformer_attention_amd as pkg
    x = make_inputs(w, sigma=1.0, seed=seed)
    rng = np.random.default_rng(seed + 1)
    dout = round_to_dtype(rng.standard_normal(w.qkv_shape), w.dtype)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t = {n: torch.from_numpy(np.ascontiguousarray(a)).to(torch.float32 if n == "bias" else tdt).to(dev)
         for n, a in x.items()}
    td = torch.from_numpy(dout).to(tdt).to(dev)
    kw = dict(grid=(w.grid_h, w.grid_w), window=w.window, prefix_tokens=w.prefix, mode=w.mode,
              terms="".join(sorted(w.terms)), map=w.map, alpha=w.alpha, beta=w.beta, gamma=w.gamma,
              rounding=w.reading, bias=t.get("bias"), rq=t.get("rq"), rk=t.get("rk"), rv=t.get("rv"),
              method=w.method)
    _, lse = pkg.rpe_attn_fwd(t["q"], t["k"], t["v"], return_lse=True, **kw)
    g = pkg.rpe_attn_bwd(t["q"], t["k"], t["v"], td, lse, **kw)
    torch.cuda.synchronize()
    ref = attention_backward(_spec(w), x["q"], x["k"], x["v"], dout, bias=x.get("bias"), rq=x.get("rq"),
                             rk=x.get("rk"), rv=x.get("rv"))
    want = {"dq", "dk", "dv"} | {"d" + n for n in ("bias", "rq", "rk", "rv") if n in x}
    assert set(g) == want
    for n in sorted(want):
        got = g[n].cpu().numpy().astype(np.float64)
        scale = max(1.0, float(np.abs(ref[n]).max()))
        err = float(np.abs(got - ref[n]).max())
        print(f"    {n}: max err {err:.3e}  (max |ref| {scale:.3e}, rel tol {REL[w.dtype]})", flush=True)
        assert np.isfinite(got).all() and err <= REL[w.dtype] * scale, (n, err, scale)


def test_backward_binding_rejects_mismatched_inputs(dev):
    # The C entry point sizes every read and write from the descriptor, so the
    # binding refuses a grid that does not match q and tables of the wrong
    # shape, dtype or device before any launch.
    import torch
    import vision_transformer_attention_amd as pkg
    w = _fit(_D.resized(batch=1, heads=2, terms=frozenset("kv")))
    x = make_inputs(w, seed=9960)
    t = {n: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).to(dev) for n, a in x.items()}
    kw = dict(grid=(w.grid_h, w.grid_w), prefix_tokens=w.prefix, mode="contextual", terms="kv", map=w.map,
              alpha=w.alpha, beta=w.beta, gamma=w.gamma, rk=t["rk"], rv=t["rv"])
    _, lse = pkg.rpe_attn_fwd(t["q"], t["k"], t["v"], return_lse=True, **kw)
    dout = torch.ones_like(t["q"])
    print("[case] backward binding rejects a grid without its class token", flush=True)
    with pytest.raises(ValueError):
        pkg.rpe_attn_bwd(t["q"], t["k"], t["v"], dout, lse, **dict(kw, prefix_tokens=0))
    print("[case] backward binding rejects tables of the wrong shape / dtype / missing", flush=True)
    with pytest.raises(ValueError):
        pkg.rpe_attn_bwd(t["q"], t["k"], t["v"], dout, lse, **dict(kw, rk=t["rk"][:, :-1]))
    with pytest.raises(ValueError):
        pkg.rpe_attn_bwd(t["q"], t["k"], t["v"], dout, lse, **dict(kw, rv=t["rv"].float()))
    with pytest.raises(ValueError):
        pkg.rpe_attn_bwd(t["q"], t["k"], t["v"], dout, lse, **dict(kw, rk=None))
    with pytest.raises(ValueError):
        pkg.rpe_attn_bwd(t["q"], t["k"], t["v"], dout, lse, **dict(kw, rk=t["rk"].cpu()))
    with pytest.raises(ValueError):
        pkg.rpe_attn_bwd(t["q"].cpu(), t["k"], t["v"], dout, lse, **kw)
    torch.cuda.synchronize()
