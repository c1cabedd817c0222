"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Bucket ids and per-axis indices must match bit-exactly; attention outputs
within 2e-2 max-abs for bf16 inputs (fp32 accumulation) and 1e-5 for fp32.
Every case prints what it runs before it touches the GPU.
"""

import math

import numpy as np
import pytest

from oracle import Spec, attention, axis_index_table, num_buckets
from oracle.attention import bucket_map_array
from vision_transformer_attention_amd.workloads import WORKLOADS, make_inputs, round_to_dtype
from random_configs import random_config

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "fp32": 1e-5}


@pytest.fixture(scope="module")
def dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vision_transformer_attention_amd as pkg
    pkg.load()
    return torch.device("cuda:0")


def say(*a):
    print("[case]", *a, flush=True)


def spec_of(w, **over):
    kw = dict(window=w.window, prefix=w.prefix, mode=w.mode, terms=w.terms, map=w.map, alpha=w.alpha,
              beta=w.beta, gamma=w.gamma, reading=w.reading, tables_per_head=w.tables_per_head,
              method=w.method)
    kw.update(over)
    return Spec(w.grid_h, w.grid_w, **kw)


def desc_of(w):
    import vision_transformer_attention_amd as pkg
    return pkg.make_desc(batch=w.batch, heads=w.heads, head_dim=w.head_dim, grid=(w.grid_h, w.grid_w),
                         window=w.window, prefix_tokens=w.prefix, dtype=w.dtype, mode=w.mode,
                         terms="".join(sorted(w.terms)), map=w.map, alpha=w.alpha, beta=w.beta,
                         gamma=w.gamma, rounding=w.reading, tables_per_head=w.tables_per_head, method=w.method)


def fit(w):
    """The workload with its table size taken from the oracle's geometry."""
    return w.resized(table_rows=num_buckets(spec_of(w))[2])


def run_gpu(w, x, dev, scale=None, return_lse=True):
    import torch
    import vision_transformer_attention_amd as pkg
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    d = {n: torch.from_numpy(np.ascontiguousarray(a)).to(torch.float32 if n == "bias" else tdt).to(dev)
         for n, a in x.items()}
    o, lse = pkg.rpe_attn_fwd(d["q"], d["k"], d["v"], grid=(w.grid_h, w.grid_w), window=w.window,
                              prefix_tokens=w.prefix, mode=w.mode, terms="".join(sorted(w.terms)),
                              map=w.map, alpha=w.alpha, beta=w.beta, gamma=w.gamma, rounding=w.reading,
                              scale=scale, bias=d.get("bias"), rq=d.get("rq"), rk=d.get("rk"),
                              rv=d.get("rv"), return_lse=True, method=w.method)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def run_oracle(w, x, scale=None, **sel):
    spec = spec_of(w, scale=scale)
    return attention(spec, x["q"], x["k"], x["v"], bias=x.get("bias"), rq=x.get("rq"), rk=x.get("rk"),
                     rv=x.get("rv"), **sel)


def compare(w, x, dev, tol=None, scale=None, **sel):
    go, gl = run_gpu(w, x, dev, scale=scale)
    ro, rl = run_oracle(w, x, scale=scale, **sel)
    mask = ~np.isnan(ro)
    assert np.isfinite(go).all(), "non-finite GPU output"
    err = float(np.abs(go - ro)[mask].max())
    lmask = ~np.isnan(rl)
    lerr = float(np.abs(gl - rl)[lmask].max())
    tol = TOL[w.dtype] if tol is None else tol
    print(f"    max|o - oracle| = {err:.3e}  max|lse - oracle| = {lerr:.3e}  (tol {tol})", flush=True)
    assert err <= tol, err
    assert lerr <= tol, lerr
    return err


_QKV_DET = WORKLOADS["deit_s_irpe_qkv"]


# ------------------------------------------------------------------------------ index + map

@pytest.mark.parametrize("abg,reading", [((1.9, 3.8, 15.2), "capped"), ((1.9, 3.8, 15.2), "trunc"),
                                         ((3.8, 7.6, 30.4), "capped"), ((3.8, 7.6, 30.4), "trunc"),
                                         ((2.0, 4.0, 16.0), "capped"), ((1.3, 5.7, 9.1), "capped"),
                                         ((3.0, 3.0, 9.0), "trunc"), ((0.5, 1.6, 5.0), "capped")])
def test_axis_index_bit_exact(dev, abg, reading):
    import vision_transformer_attention_amd as pkg
    a, b, g = abg
    say("axis_index", abg, reading)
    d = pkg.make_desc(mode="contextual", terms="k", map="piecewise", alpha=a, beta=b, gamma=g,
                      rounding=reading, grid=(64, 64))
    got = pkg.rpe_attn_axis_index(d, 200, device=dev).cpu().numpy().tolist()
    assert got == axis_index_table(200, a, b, g, reading)


MAP_CASES = [(name, reading) for name in WORKLOADS for reading in ("capped", "trunc")
             if WORKLOADS[name].map in ("piecewise", "swin") and (WORKLOADS[name].map == "piecewise" or reading == "capped")]


@pytest.mark.parametrize("name,reading", MAP_CASES)
def test_bucket_map_bit_exact(dev, name, reading):
    import vision_transformer_attention_amd as pkg
    w = WORKLOADS[name].resized(reading=reading)
    say("bucket_map", name, reading)
    got = pkg.rpe_attn_bucket_map(desc_of(w), device=dev).cpu().numpy()
    ref = bucket_map_array(spec_of(w))
    assert got.dtype == np.int16 and got.shape == ref.shape
    assert (got.astype(np.int64) == ref).all()


@pytest.mark.parametrize("m", ["euclidean", "euclidean_rounded", "quantized", "quantized_squared"])
@pytest.mark.parametrize("gh,gw,window,prefix,abg", [(14, 14, 0, 1, (1.9, 3.8, 15.2)),
                                                     (9, 23, 0, 0, (1.0, 2.0, 8.0)),
                                                     (14, 14, 7, 0, (1.9, 3.8, 15.2)),
                                                     (91, 91, 0, 0, (3.8, 7.6, 30.4)),
                                                     (2, 127, 0, 1, (1.9, 3.8, 15.2))])
def test_undirected_pair_rows_bit_exact(dev, m, gh, gw, window, prefix, abg):
    # Under an undirected map the bucket map names each pair's table row
    # u(dy, dx) + H (iRPE page, Method, eqs. 19-21), evaluated on the device in
    # float64; the oracle evaluates each distinct offset on its own.  91 x 91 is
    # the largest square grid the device tabulation takes ((R-1)^2 + (C-1)^2 <
    # 16384), 2 x 127 the widest two-row one.
    import vision_transformer_attention_amd as pkg
    from oracle.attention import pair_rows_arrays
    a, b, g = abg
    say("undirected pair rows", m, gh, gw, window, prefix, abg)
    spec = Spec(gh, gw, window=window, prefix=prefix, mode="bias", map=m, alpha=a, beta=b, gamma=g)
    d = pkg.make_desc(grid=(gh, gw), window=window, prefix_tokens=prefix, mode="bias", map=m, alpha=a, beta=b,
                      gamma=g)
    got = pkg.rpe_attn_bucket_map(d, device=dev).cpu().numpy().astype(np.int64)
    if gh * gw > 4096:
        # sampled rows of the oracle's map: every offset of the grid appears in
        # the rows of the four corner tokens
        t = gh * gw
        rows = [0, gw - 1, t - gw, t - 1, t // 2]
        ref = _undirected_rows(spec, rows)
        assert (got[rows] == ref).all()
    else:
        (ref,) = pair_rows_arrays(spec)
        assert (got == ref).all()


def _undirected_rows(spec, rows):
    from oracle import num_buckets
    h, _, _ = num_buckets(spec)
    gw, t = spec.grid_w, spec.grid_h * spec.grid_w
    out = np.empty((len(rows), t), dtype=np.int64)
    cache = {}
    for r, i in enumerate(rows):
        for j in range(t):
            key = (abs(i // gw - j // gw), abs(i % gw - j % gw))
            if key not in cache:
                cache[key] = spec.u(*key) + h
            out[r, j] = cache[key]
    return out


@pytest.mark.parametrize("gh,gw,window,prefix", [(1, 1, 0, 0), (3, 7, 0, 2), (9, 4, 0, 1), (6, 6, 3, 0),
                                                 (8, 12, 4, 0), (5, 5, 0, 16)])
def test_bucket_map_shapes(dev, gh, gw, window, prefix):
    import vision_transformer_attention_amd as pkg
    say("bucket_map shape", gh, gw, window, prefix)
    for mode, mp in (("bias", "swin"), ("contextual", "piecewise")):
        if mp == "swin" and prefix:
            continue
        spec = Spec(gh, gw, window=window, prefix=prefix, mode=mode, terms={"k"} if mode == "contextual" else set(),
                    map=mp, alpha=1.2, beta=2.9, gamma=7.0)
        d = pkg.make_desc(grid=(gh, gw), window=window, prefix_tokens=prefix, mode=mode,
                          terms="k" if mode == "contextual" else "", map=mp, alpha=1.2, beta=2.9, gamma=7.0)
        got = pkg.rpe_attn_bucket_map(d, device=dev).cpu().numpy().astype(np.int64)
        assert (got == bucket_map_array(spec)).all()


# ------------------------------------------------------------------------------ attention

SMALL = {
    "swin_tiny": WORKLOADS["swin_tiny"],
    "swin_t_w7": WORKLOADS["swin_t_w7"].resized(batch=2, heads=3, grid_h=14, grid_w=21),
    "deit_s_irpe_k": WORKLOADS["deit_s_irpe_k"].resized(batch=2, heads=2),
    "deit_s_irpe_qkv": WORKLOADS["deit_s_irpe_qkv"].resized(batch=2, heads=2),
    "highres_irpe_k": WORKLOADS["highres_irpe_k"].resized(batch=1, heads=1, grid_h=24, grid_w=56),
}


@pytest.mark.parametrize("sigma", [0.02, 1.0])
@pytest.mark.parametrize("name", list(SMALL))
def test_parity_small(dev, name, sigma):
    w = SMALL[name]
    say("parity", name, w.qkv_shape, "sigma", sigma)
    compare(w, make_inputs(w, sigma=sigma), dev)


@pytest.mark.parametrize("name", ["swin_t_w7", "deit_s_irpe_k", "deit_s_irpe_qkv", "highres_irpe_k"])
def test_parity_fp32(dev, name):
    # fp32 reruns of the bf16 workload shapes, at the fp32 tolerance
    w = SMALL[name].resized(dtype="fp32")
    if name == "highres_irpe_k":
        w = w.resized(grid_h=12)
    say("parity fp32", name, w.qkv_shape)
    compare(w, make_inputs(w, sigma=1.0, seed=3000 + w.index), dev)


def test_isolation_terms(dev):
    # k = 0: logits are the position terms alone; v = 0: the output is the value term alone.
    w = SMALL["deit_s_irpe_qkv"]
    x = make_inputs(w, sigma=1.0, seed=4000)
    say("isolation k=0", w.qkv_shape)
    x0 = dict(x, k=np.zeros_like(x["k"]))
    compare(w, x0, dev)
    say("isolation v=0", w.qkv_shape)
    x1 = dict(x, v=np.zeros_like(x["v"]))
    compare(w, x1, dev)
    say("isolation q=0", w.qkv_shape)
    compare(w, dict(x, q=np.zeros_like(x["q"])), dev)


TERMS = ["k", "q", "v", "kq", "kv", "qv", "kqv"]


@pytest.mark.parametrize("terms", TERMS)
@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 32), ("fp32", 16), ("bf16", 16)])
def test_term_combinations(dev, terms, dtype, d):
    w = WORKLOADS["deit_s_irpe_qkv"].resized(batch=1, heads=2, head_dim=d, grid_h=7, grid_w=9,
                                             terms=frozenset(terms), dtype=dtype)
    say("terms", terms, dtype, d, w.qkv_shape)
    compare(w, make_inputs(w, sigma=1.0, seed=5000), dev)


EDGE = [
    # (label, overrides on the DeiT QKV workload)
    ("grid 1x1 + cls", dict(grid_h=1, grid_w=1)),
    ("grid 1x1 no cls", dict(grid_h=1, grid_w=1, prefix=0)),
    ("no cls 5x11", dict(grid_h=5, grid_w=11, prefix=0)),
    ("prefix block (no room in the padded row)", dict(grid_h=4, grid_w=16, prefix=1)),
    ("prefix 3 in tail", dict(grid_h=5, grid_w=13, prefix=3)),
    ("prefix 16 block", dict(grid_h=3, grid_w=5, prefix=16)),
    ("two subtiles per row", dict(grid_h=3, grid_w=27, prefix=1)),
    ("four subtiles per row", dict(grid_h=2, grid_w=61, prefix=1)),
    ("width 8", dict(grid_h=9, grid_w=8, prefix=1)),
    ("width 3", dict(grid_h=11, grid_w=3, prefix=2)),
    ("trunc reading", dict(reading="trunc")),
    ("per-head tables", dict(tables_per_head=True, heads=3)),
    ("odd tokens 17x17", dict(grid_h=17, grid_w=17, alpha=2.0, beta=4.0, gamma=16.0)),
]


@pytest.mark.parametrize("terms", ["kqv", "k"])
@pytest.mark.parametrize("label,over", EDGE)
def test_edge_shapes(dev, label, over, terms):
    # "k" alone keeps the per-row key scores in fp16; with the value term they are fp32
    base = dict(batch=2, heads=2, grid_h=6, grid_w=7, terms=frozenset(terms))
    base.update(over)
    w = fit(WORKLOADS["deit_s_irpe_qkv"].resized(**base))
    say("edge", label, terms, w.qkv_shape)
    compare(w, make_inputs(w, sigma=1.0, seed=6000), dev)


SWIN_EDGE = [
    ("window 2", dict(grid_h=6, grid_w=8, window=2)),
    ("window 3", dict(grid_h=9, grid_w=6, window=3)),
    ("window 5", dict(grid_h=10, grid_w=15, window=5)),
    ("window 8", dict(grid_h=16, grid_w=8, window=8)),
    ("window 9 (wide rows)", dict(grid_h=9, grid_w=18, window=9)),
    ("shared bias", dict(tables_per_head=False)),
    ("global swin map", dict(grid_h=5, grid_w=6, window=0)),
    ("fp32 d32", dict(dtype="fp32")),
    ("d64", dict(head_dim=64)),
]


@pytest.mark.parametrize("label,over", SWIN_EDGE)
def test_swin_edge(dev, label, over):
    base = dict(batch=2, heads=2, grid_h=14, grid_w=14)
    base.update(over)
    w = fit(WORKLOADS["swin_t_w7"].resized(**base))
    say("swin edge", label, w.qkv_shape)
    compare(w, make_inputs(w, sigma=1.0, seed=7000), dev)


# Mode and mapping variants on the same kernel: the iRPE bias mode on a global
# grid with the piecewise index (shared or per-head table, with and without a
# class token), and contextual terms inside Swin windows (both maps).
_D = WORKLOADS["deit_s_irpe_k"]
MODE_VARIANTS = [
    ("iRPE bias, global 14x14 + cls, shared table", _D.resized(batch=2, heads=3, mode="bias", terms=frozenset())),
    ("iRPE bias, global 14x14 + cls, per-head tables",
     _D.resized(batch=2, heads=3, mode="bias", terms=frozenset(), tables_per_head=True)),
    ("iRPE bias, global 9x13 no cls, trunc reading",
     _D.resized(batch=2, heads=2, grid_h=9, grid_w=13, prefix=0, mode="bias", terms=frozenset(), reading="trunc")),
    ("iRPE bias fp32 d32, global 10x10 + 2 prefix",
     _D.resized(batch=2, heads=2, head_dim=32, grid_h=10, grid_w=10, prefix=2, mode="bias", terms=frozenset(),
                dtype="fp32")),
    ("iRPE bias, wide 12x40 global grid", WORKLOADS["highres_irpe_k"].resized(batch=1, heads=2, grid_h=12,
                                                                             grid_w=40, mode="bias",
                                                                             terms=frozenset())),
    ("contextual K in 7x7 windows, piecewise", _D.resized(batch=2, heads=2, grid_h=14, grid_w=21, window=7,
                                                          prefix=0)),
    ("contextual QKV in 7x7 windows, piecewise",
     _D.resized(batch=2, heads=2, grid_h=14, grid_w=14, window=7, prefix=0, terms=frozenset("kqv"))),
    ("contextual QKV in 7x7 windows, Swin map, per-head tables",
     _D.resized(batch=2, heads=3, head_dim=32, grid_h=14, grid_w=14, window=7, prefix=0, terms=frozenset("kqv"),
                map="swin", tables_per_head=True)),
    ("contextual K in 4x4 windows fp32 d16",
     _D.resized(batch=2, heads=2, head_dim=16, grid_h=8, grid_w=12, window=4, prefix=0, dtype="fp32")),
]


# Variable resolution: the DeiT-S key term over the grids of 112^2 .. 384^2 inputs
# (7x7 .. 24x24 patches + cls) and DETR-like non-square grids; every grid gets its
# own thresholds, key-slot layout and launch plan.
RESOLUTIONS = [(7, 7), (10, 10), (18, 18), (24, 24), (9, 38), (17, 25)]


@pytest.mark.parametrize("gh,gw", RESOLUTIONS)
def test_resolution_sweep(dev, gh, gw):
    w = fit(_D.resized(batch=2, heads=2, grid_h=gh, grid_w=gw, prefix=1 if gh == gw else 0))
    say("resolution", gh, gw, w.qkv_shape)
    compare(w, make_inputs(w, sigma=1.0, seed=9800 + gh * 100 + gw), dev)


@pytest.mark.parametrize("label,w", MODE_VARIANTS)
def test_mode_variants(dev, label, w):
    w = fit(w)
    say("mode variant", label, w.qkv_shape)
    compare(w, make_inputs(w, sigma=1.0, seed=9500), dev)


# The Cross mapping: Cross tables (row-offset half, column-offset half) are
# rewritten as Product tables by rpe_attn_cross_to_product, then the Product
# forward runs.  The conversion is checked exactly against its definition, the
# attention against the oracle's own Cross mapping.
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_cross_to_product_exact(dev, dtype):
    import torch
    import vision_transformer_attention_amd as pkg
    say("cross_to_product", dtype)
    tdt = torch.float32 if dtype == "fp32" else torch.bfloat16
    d = pkg.make_desc(batch=1, heads=3, head_dim=32, grid=(14, 14), prefix_tokens=1, dtype=dtype,
                      mode="contextual", terms="kqv", map="piecewise", alpha=1.9, beta=3.8, gamma=15.2,
                      tables_per_head=True)
    _, s, nb = pkg.rpe_attn_num_buckets(d)
    rng = np.random.default_rng(31)
    cross = torch.from_numpy(rng.standard_normal((3, 2 * s, 32)).astype(np.float32)).to(tdt)
    got = pkg.rpe_attn_cross_to_product(d, cross.to(dev)).cpu()
    torch.cuda.synchronize()
    c32 = cross.float()
    by, bx = np.arange(nb) // s, s + np.arange(nb) % s
    ref = (c32[:, by] + c32[:, bx]).to(tdt)          # one fp32 sum, one rounding
    assert got.dtype == tdt and tuple(got.shape) == (3, nb, 32)
    assert torch.equal(got, ref)
    db = pkg.make_desc(batch=1, heads=3, head_dim=32, grid=(7, 7), window=7, mode="bias", map="swin")
    _, s, nb = pkg.rpe_attn_num_buckets(db)
    cb = torch.from_numpy(rng.standard_normal((1, 2 * s)).astype(np.float32))
    got = pkg.rpe_attn_cross_to_product(db, cb.to(dev)).cpu()
    by, bx = np.arange(nb) // s, s + np.arange(nb) % s
    assert torch.equal(got, cb[:, by] + cb[:, bx])


CROSS_CASES = [
    ("cross bias, global 14x14 + cls", _D.resized(batch=2, heads=3, mode="bias", terms=frozenset(),
                                                  method="cross")),
    ("cross bias, Swin 7x7 windows, per-head", WORKLOADS["swin_t_w7"].resized(batch=2, heads=3, grid_h=14,
                                                                             grid_w=14, tables_per_head=True,
                                                                             method="cross")),
    ("cross contextual K, global 14x14 + cls", _D.resized(batch=2, heads=2, method="cross")),
    ("cross contextual KQV, global 14x14 + cls", _D.resized(batch=2, heads=2, terms=frozenset("kqv"),
                                                            method="cross")),
    ("cross contextual QV, 9x13 no cls, per-head tables, d32",
     _D.resized(batch=2, heads=3, head_dim=32, grid_h=9, grid_w=13, prefix=0, terms=frozenset("qv"),
                tables_per_head=True, method="cross")),
    ("cross contextual KQV, rows of 4 (per-bucket value sums), 11x3 + 2 prefix",
     _D.resized(batch=2, heads=2, grid_h=11, grid_w=3, prefix=2, terms=frozenset("kqv"), method="cross")),
    ("cross contextual QKV fp32 d16, 7x7 windows",
     _D.resized(batch=2, heads=2, head_dim=16, grid_h=14, grid_w=14, window=7, prefix=0, terms=frozenset("kqv"),
                dtype="fp32", method="cross")),
    ("cross contextual K, wide 10x40 grid", WORKLOADS["highres_irpe_k"].resized(batch=1, heads=2, grid_h=10,
                                                                               grid_w=40, method="cross")),
    ("cross contextual KV, wide 6x61 grid + cls", _D.resized(batch=1, heads=2, grid_h=6, grid_w=61,
                                                             terms=frozenset("kv"), method="cross")),
    ("cross contextual K, 17 per axis (beta 7.6), 24x24 grid",
     WORKLOADS["highres_irpe_k"].resized(batch=1, heads=2, grid_h=24, grid_w=24, method="cross")),
    ("cross contextual KQV, trunc reading", _D.resized(batch=1, heads=2, terms=frozenset("kqv"), reading="trunc",
                                                       method="cross")),
]


@pytest.mark.parametrize("label,w", CROSS_CASES)
def test_cross_mapping(dev, label, w):
    # Cross tables (2S rows) go to the forward as they are and are held to the
    # oracle's own Cross mapping (iRPE page, Method, eqs. 22-24: the sum of a
    # row-offset and a column-offset encoding per pair) at the usual tolerance.
    w = fit(w)
    say("cross", label, w.qkv_shape, "table rows", w.table_rows)
    compare(w, make_inputs(w, sigma=1.0, seed=9700), dev)


def test_cross_full_size(dev):
    # the DeiT-S Cross workload at full size, sigma = 1 tables, sampled (b, h)
    w = WORKLOADS["deit_s_irpe_k_cross"].resized(terms=frozenset("kqv"))
    say("cross full size KQV", w.qkv_shape, "sampled (b, h): [5, 60], [1, 4]")
    compare(w, make_inputs(w, sigma=1.0), dev, batch_sel=[5, 60], heads_sel=[1, 4])


# Strided views: q, k, v as the three slices of one fused [B, N, 3, H, d]
# projection and o written into a [B, N, H, d] tensor, with no copies.
STRIDED = [
    ("DeiT-S K, fused qkv", _D.resized(batch=2, heads=3)),
    ("DeiT-S KQV d32, fused qkv", _D.resized(batch=2, heads=3, head_dim=32, terms=frozenset("kqv"))),
    ("Swin W7 bias, fused qkv", WORKLOADS["swin_t_w7"].resized(batch=2, heads=3, grid_h=14, grid_w=21)),
    ("wide 5x40 K fp32 d16, fused qkv", WORKLOADS["highres_irpe_k"].resized(batch=2, heads=2, head_dim=16,
                                                                           grid_h=5, grid_w=40, dtype="fp32")),
    ("4x4 windows bias fp32 d16 (several windows per workgroup)",
     WORKLOADS["swin_tiny"].resized(batch=3, heads=4, grid_h=64, grid_w=64)),
]


@pytest.mark.parametrize("label,w", STRIDED)
def test_strided_views(dev, label, w):
    import torch
    import vision_transformer_attention_amd as pkg
    w = fit(w)
    x = make_inputs(w, sigma=1.0, seed=9600)
    say("strided", label, w.qkv_shape)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    B, H, N, d = w.qkv_shape
    fused = torch.empty((B, N, 3, H, d), dtype=tdt)
    for i, n in enumerate("qkv"):
        fused[:, :, i] = torch.from_numpy(x[n]).to(tdt).permute(0, 2, 1, 3)
    fused = fused.to(dev)
    q, k, v = (fused[:, :, i].permute(0, 2, 1, 3) for i in range(3))
    assert not q.is_contiguous()
    o_buf = torch.full((B, N, H, d), float("nan"), dtype=tdt, device=dev)
    o = o_buf.permute(0, 2, 1, 3)
    t = {n: torch.from_numpy(np.ascontiguousarray(a)).to(torch.float32 if n == "bias" else tdt).to(dev)
         for n, a in x.items() if n not in "qkv"}
    _, lse = pkg.rpe_attn_fwd(q, k, v, grid=(w.grid_h, w.grid_w), window=w.window, prefix_tokens=w.prefix,
                              mode=w.mode, terms="".join(sorted(w.terms)), map=w.map, alpha=w.alpha, beta=w.beta,
                              gamma=w.gamma, rounding=w.reading, bias=t.get("bias"), rq=t.get("rq"),
                              rk=t.get("rk"), rv=t.get("rv"), out=o, return_lse=True)
    torch.cuda.synchronize()
    go = o.float().cpu().numpy().astype(np.float64)
    sel = dict(batch_sel=[0, B - 1], heads_sel=[0, H - 1])
    if w.window:
        sel["units"] = [0, 1, 255] if w.grid_h == 64 else None
    ro, rl = run_oracle(w, x, **sel)
    mask = ~np.isnan(ro)
    err = float(np.abs(go - ro)[mask].max())
    lerr = float(np.abs(lse.cpu().numpy() - rl)[~np.isnan(rl)].max())
    print(f"    max|o - oracle| = {err:.3e}  lse {lerr:.3e}", flush=True)
    assert np.isfinite(go).all(), "o rows left unwritten or non-finite"
    assert err <= TOL[w.dtype] and lerr <= TOL[w.dtype], (err, lerr)


# Undirected maps (Euclidean, Quantization; page and code readings).  The forward
# takes their table of S rows as it is: a per-offset index table gathers the row
# in two steps.  rpe_attn_undirected_to_product, which expands that table into
# the Swin map's table over raw offsets, is checked exactly (it copies rows
# chosen by indices computed on the device in fp64).
UND_MAPS = ["euclidean", "euclidean_rounded", "quantized", "quantized_squared"]


def _expanded_reference(spec, table):
    """[T, S'^2(, d)] with row (dy + H') S' + dx + H' = table[u(dy, dx) + H] (oracle index)."""
    r, c = spec.unit_side
    hp = max(r, c) - 1
    sp = 2 * hp + 1
    h, _, _ = num_buckets(spec)
    out = np.zeros((table.shape[0], sp * sp) + table.shape[2:])
    for dy in range(-(r - 1), r):
        for dx in range(-(c - 1), c):
            out[:, (dy + hp) * sp + dx + hp] = table[:, spec.u(dy, dx) + h]
    return out


@pytest.mark.parametrize("m", UND_MAPS)
@pytest.mark.parametrize("gh,gw,window,reading", [(14, 14, 0, "capped"), (9, 13, 0, "trunc"), (56, 56, 7, "capped"),
                                                  (40, 40, 0, "capped")])
def test_undirected_expansion_exact(dev, m, gh, gw, window, reading):
    import torch
    import vision_transformer_attention_amd as pkg
    abg = (1.9, 3.8, 15.2) if gh < 40 else (3.8, 7.6, 30.4)
    say("undirected expansion", m, gh, gw, window, reading)
    d = pkg.make_desc(batch=1, heads=2, head_dim=16, grid=(gh, gw), window=window, mode="bias", map=m,
                      alpha=abg[0], beta=abg[1], gamma=abg[2], rounding=reading, tables_per_head=True)
    spec = Spec(gh, gw, window=window, mode="bias", map=m, alpha=abg[0], beta=abg[1], gamma=abg[2], reading=reading)
    _, s, rows = pkg.rpe_attn_num_buckets(d)
    tab = np.arange(2 * rows, dtype=np.float32).reshape(2, rows) + 1.0     # distinct rows
    got = pkg.rpe_attn_undirected_to_product(d, torch.from_numpy(tab).to(dev)).cpu().numpy()
    torch.cuda.synchronize()
    ref = _expanded_reference(spec, tab.astype(np.float64))
    assert got.shape == ref.shape
    assert (got == ref).all(), np.argwhere(got != ref)[:5]


_UND = [
    ("bias, global 14x14 + cls", _D.resized(batch=2, heads=3, mode="bias", terms=frozenset(), tables_per_head=True)),
    ("contextual K, 7x7 windows", _D.resized(batch=2, heads=2, grid_h=14, grid_w=21, window=7, prefix=0)),
    ("contextual KQV, 7x7 windows, d32", _D.resized(batch=2, heads=2, head_dim=32, grid_h=14, grid_w=14, window=7,
                                                    prefix=0, terms=frozenset("kqv"))),
    ("contextual K, global 14x14 + cls", _D.resized(batch=1, heads=2)),
    ("contextual QV fp32 d16, 4x4 windows", _D.resized(batch=2, heads=2, head_dim=16, grid_h=8, grid_w=12,
                                                       window=4, prefix=0, terms=frozenset("qv"), dtype="fp32")),
]


@pytest.mark.parametrize("m", UND_MAPS)
@pytest.mark.parametrize("label,w", _UND)
def test_undirected_maps(dev, m, label, w):
    w = fit(w.resized(map=m))
    say("undirected", m, label, w.qkv_shape, "table rows", w.table_rows)
    compare(w, make_inputs(w, sigma=1.0, seed=9900), dev)


# Units too large for a table over raw offsets to stay in LDS: 32x32 and 56x56
# global grids (63x63 and 111x111 offsets), sampled over batch and heads.
_UND_LARGE = [
    ("contextual K, global 32x32 + cls", "euclidean",
     _D.resized(batch=2, heads=2, grid_h=32, grid_w=32)),
    ("contextual KQV, global 32x32 + cls", "quantized",
     _D.resized(batch=1, heads=2, grid_h=32, grid_w=32, terms=frozenset("kqv"))),
    ("contextual KV fp32 d32, global 24x40", "quantized_squared",
     _D.resized(batch=1, heads=2, head_dim=32, grid_h=24, grid_w=40, prefix=0, terms=frozenset("kv"),
                dtype="fp32")),
    ("bias, global 56x56 + cls", "euclidean_rounded",
     _D.resized(batch=1, heads=3, grid_h=56, grid_w=56, mode="bias", terms=frozenset(), tables_per_head=True,
                alpha=3.8, beta=7.6, gamma=30.4)),
    ("contextual QV, 28x28 windows on 56x56", "euclidean",
     _D.resized(batch=1, heads=2, grid_h=56, grid_w=56, window=28, prefix=0, terms=frozenset("qv"))),
]


@pytest.mark.parametrize("label,m,w", _UND_LARGE)
def test_undirected_large_units(dev, label, m, w):
    w = fit(w.resized(map=m))
    say("undirected large", m, label, w.qkv_shape, "table rows", w.table_rows)
    sel = dict(batch_sel=[w.batch - 1], heads_sel=[w.heads - 1])
    if w.window:
        sel["units"] = [0, 3]
    compare(w, make_inputs(w, sigma=1.0, seed=9950), dev, **sel)


# Units more than 64 columns wide: grid rows padded to a multiple of 32 key
# slots (96 to 256 here) span 3 to 8 key blocks, whose column parts are refilled
# per block (a 50x84 detection-style grid, C = 65 just past 64, C = 96 with no
# padding left for the class token, C = 256 the widest).  (Swin-map
# units that wide need more LDS than a CU has: their tables have (2C-1)^2 rows.)
_WIDE_ROWS = [
    ("contextual K, 6x84 + cls", _D.resized(batch=2, heads=2, grid_h=6, grid_w=84)),
    ("contextual KQV, 5x100 + cls", _D.resized(batch=1, heads=2, grid_h=5, grid_w=100, terms=frozenset("kqv"))),
    ("contextual KQV fp32 d32, 4x130", _D.resized(batch=1, heads=2, head_dim=32, grid_h=4, grid_w=130, prefix=0,
                                                  terms=frozenset("kqv"), dtype="fp32")),
    ("contextual QV d16, 7x65 + cls", _D.resized(batch=2, heads=2, head_dim=16, grid_h=7, grid_w=65,
                                                 terms=frozenset("qv"))),
    ("contextual KQ d32, 2x256 + cls", _D.resized(batch=1, heads=2, head_dim=32, grid_h=2, grid_w=256,
                                                  terms=frozenset("kq"))),
    ("iRPE bias, 3x200 + 2 prefix in the row padding, per-head tables",
     _D.resized(batch=1, heads=3, grid_h=3, grid_w=200, prefix=2, mode="bias", terms=frozenset(),
                tables_per_head=True)),
    ("no position terms fp32, 4x150 + cls", _D.resized(batch=1, heads=2, grid_h=4, grid_w=150, mode="none",
                                                       terms=frozenset(), map="swin", dtype="fp32")),
    ("cross contextual KV, 5x96 + cls", _D.resized(batch=1, heads=2, grid_h=5, grid_w=96, terms=frozenset("kv"),
                                                   method="cross")),
    ("euclidean contextual KQV, 6x90", _D.resized(batch=1, heads=2, grid_h=6, grid_w=90, prefix=0,
                                                  terms=frozenset("kqv"), map="euclidean")),
    ("contextual V, 3x70 + cls", _D.resized(batch=2, heads=2, grid_h=3, grid_w=70, terms=frozenset("v"))),
    ("contextual K, 50x84 detection grid", _D.resized(batch=1, heads=2, grid_h=50, grid_w=84, prefix=0)),
    ("contextual K, 72x72 windows on a 72x144 grid", _D.resized(batch=1, heads=1, grid_h=72, grid_w=144,
                                                                window=72, prefix=0)),
]


@pytest.mark.parametrize("label,w", _WIDE_ROWS)
def test_wide_rows(dev, label, w):
    w = fit(w) if w.mode != "none" else w
    sel = {}
    if w.grid_h * w.grid_w > 2000:
        sel = dict(batch_sel=[w.batch - 1], heads_sel=[w.heads - 1])
        if w.window:
            sel["units"] = [1]
    say("wide rows", label, w.qkv_shape, "sampled" if sel else "")
    compare(w, make_inputs(w, sigma=1.0, seed=9960), dev, **sel)


@pytest.mark.parametrize("i", range(24))
def test_random_configs(dev, i):
    w = random_config(i)
    say("random config", i, w.qkv_shape, w.mode, "".join(sorted(w.terms)), w.map, w.method, w.dtype,
        "grid", (w.grid_h, w.grid_w), "window", w.window, "prefix", w.prefix, "per-head", w.tables_per_head)
    compare(w, make_inputs(w, sigma=1.0, seed=12500 + i), dev)


def test_no_position_mode(dev):
    import torch
    import vision_transformer_attention_amd as pkg
    w = WORKLOADS["deit_s_irpe_k"].resized(batch=2, heads=2, mode="none", terms=frozenset(), map="swin")
    x = make_inputs(w, seed=8000)
    say("mode none", w.qkv_shape)
    q, k, v = (torch.from_numpy(x[n]).to(torch.bfloat16).to(dev) for n in "qkv")
    o = pkg.rpe_attn_fwd(q, k, v, grid=(14, 14), prefix_tokens=1, mode="none")
    torch.cuda.synchronize()
    ref, _ = attention(Spec(14, 14, prefix=1, mode="none"), x["q"], x["k"], x["v"])
    err = float(np.abs(o.float().cpu().numpy() - ref).max())
    print(f"    max err {err:.3e}", flush=True)
    assert err <= 2e-2


def test_explicit_scale(dev):
    w = SMALL["deit_s_irpe_qkv"]
    say("explicit scale 0.05", w.qkv_shape)
    compare(w, make_inputs(w, sigma=1.0, seed=9000), dev, scale=0.05)
    w = SMALL["swin_t_w7"]
    say("explicit scale 0.3 swin", w.qkv_shape)
    compare(w, make_inputs(w, sigma=1.0, seed=9001), dev, scale=0.3)


def test_shaw_page_example_on_gpu(dev):
    # The Shaw-style page's layer as a 1 x 6 grid with clip 3, zero-padded from d = 4 to 16
    # (padding adds zero products), scale 1/sqrt(4) given explicitly; fp32.
    import test_oracle_attention as toa
    q, k, v, a_k, a_v = toa._shaw_page_setup()
    spec, rk, rv = toa._shaw_as_2d(a_k, a_v)
    pad = lambda a: np.concatenate([a, np.zeros(a.shape[:-1] + (12,))], axis=-1)
    x = {"q": round_to_dtype(pad(q)[None, None], "fp32"), "k": round_to_dtype(pad(k)[None, None], "fp32"),
         "v": round_to_dtype(pad(v)[None, None], "fp32"), "rk": round_to_dtype(pad(rk), "fp32"),
         "rv": round_to_dtype(pad(rv), "fp32")}
    w = WORKLOADS["deit_s_irpe_k"].resized(batch=1, heads=1, head_dim=16, grid_h=1, grid_w=6, prefix=0,
                                           terms=frozenset("kv"), alpha=3.0, beta=3.0, gamma=10.0,
                                           dtype="fp32", table_rows=rk.shape[1])
    say("shaw page example", w.qkv_shape)
    compare(w, x, dev, scale=0.5)


def test_empty_batch(dev):
    import torch
    import vision_transformer_attention_amd as pkg
    say("empty batch")
    q = torch.zeros((0, 2, 197, 64), dtype=torch.bfloat16, device=dev)
    rk = torch.zeros((1, 81, 64), dtype=torch.bfloat16, device=dev)
    o = pkg.rpe_attn_fwd(q, q, q, grid=(14, 14), prefix_tokens=1, mode="contextual", terms="k",
                         map="piecewise", alpha=1.9, beta=3.8, gamma=15.2, rk=rk)
    torch.cuda.synchronize()
    assert o.shape == q.shape


# Keys whose logits climb steeply along the key stream: the running maximum
# starts at the first block's and has to move several times (by more than 2^64
# in the weights), rescaling O, the row sum and the value-term weight sums
# mid-stream.  Every query gets +4 along the all-ones direction and each key
# ramp * (row / (rows - 1) - 1) along it (row within the unit; prefix keys as
# row 0), so the logits climb by about 4 * ramp * sqrt(d) to values near 0 at
# the last key row: the weights that matter come from logits of ordinary size.
_QKV = WORKLOADS["deit_s_irpe_qkv"]
RAMP_CASES = [
    ("DeiT-S QKV 14x14 + cls (per-column weight sums)", _QKV.resized(batch=1, heads=2), 5.0),
    ("QKV 7x7 windows (per-column sums, rows of 8)",
     _QKV.resized(batch=1, heads=2, grid_h=14, grid_w=14, window=7, prefix=0), 5.0),
    ("QKV 9x27 + cls (per-column sums, rows of 32)", _QKV.resized(batch=1, heads=2, grid_h=9, grid_w=27), 5.0),
    ("QKV 11x3 + 2 prefix (per-bucket sums, rows of 4)",
     _QKV.resized(batch=1, heads=2, grid_h=11, grid_w=3, prefix=2), 5.0),
    ("QKV 3x61 + cls (per-bucket sums, wide rows)", _QKV.resized(batch=1, heads=2, grid_h=3, grid_w=61), 5.0),
    ("V only 14x14 + cls", _QKV.resized(batch=1, heads=2, terms=frozenset("v")), 5.0),
    ("QKV fp32 d32 10x10 + cls", _QKV.resized(batch=1, heads=2, head_dim=32, grid_h=10, grid_w=10,
                                              dtype="fp32"), 3.0),
]


@pytest.mark.parametrize("label,w,ramp", RAMP_CASES)
def test_running_max_moves(dev, label, w, ramp):
    w = fit(w)
    x = make_inputs(w, seed=9200)
    rows = w.window or w.grid_h
    y = np.arange(w.grid_h * w.grid_w) // w.grid_w
    yy = (y % w.window) if w.window else y
    t = np.concatenate([np.full(w.prefix, -ramp), ramp * (yy / max(rows - 1, 1) - 1.0)])
    x["q"] = round_to_dtype(x["q"] + 4.0, w.dtype)
    x["k"] = round_to_dtype(x["k"] + t[None, None, :, None], w.dtype)
    say("running max moves", label, w.qkv_shape)
    compare(w, x, dev)


DETERMINISM = [
    ("per-column value sums, 14x14 + cls", SMALL["deit_s_irpe_qkv"]),
    # the per-bucket layout with LDS float atomics: rows of 4 padded columns and wide rows
    ("atomic value sums, rows of 4, 11x3 + 2 prefix", _QKV_DET.resized(batch=2, heads=2, grid_h=11, grid_w=3,
                                                                        prefix=2)),
    ("atomic value sums, wide rows, 3x61 + cls", _QKV_DET.resized(batch=2, heads=2, grid_h=3, grid_w=61)),
    ("bias, several windows per workgroup", WORKLOADS["swin_t_w7"].resized(batch=8, heads=3)),
]


@pytest.mark.parametrize("label,w", DETERMINISM)
def test_deterministic(dev, label, w):
    # two calls on the same inputs give bit-identical outputs and log-sum-exps
    w = fit(w)
    x = make_inputs(w, sigma=1.0, seed=9100)
    say("determinism", label, w.qkv_shape)
    a, la = run_gpu(w, x, dev)
    b, lb = run_gpu(w, x, dev)
    assert (a == b).all() and (la == lb).all()


# ------------------------------------------------------------------------------ full sizes

# Shapes with more small windows than resident workgroups: the planner then has
# each workgroup walk several consecutive windows of one (batch, head), taking
# each window's queries through the load ring.  (label, workload, batch, head
# and window samples checked against the oracle)
_SW = WORKLOADS["swin_t_w7"]
MULTI_UNIT = [
    ("bias, 4x4 windows, 2 per workgroup", _SW.resized(batch=3, heads=4, grid_h=64, grid_w=64, window=4),
     [0, 2], [0, 3], [0, 1, 2, 3, 130, 255]),
    ("no position, 4x4 windows", _SW.resized(batch=3, heads=4, grid_h=64, grid_w=64, window=4, mode="none",
                                             map="swin"), [1], [0, 2], [0, 1, 77, 255]),
    ("fp32 d16 bias, 4x4 windows", WORKLOADS["swin_tiny"].resized(batch=3, heads=4, grid_h=64, grid_w=64),
     [0, 2], [1, 3], [0, 1, 200, 255]),
    ("bias, 8x8 windows (two key blocks)", _SW.resized(batch=16, heads=3, grid_h=64, grid_w=64, window=8),
     [0, 15], [0, 2], [0, 1, 2, 3, 62, 63]),
    ("bias, 10x10 windows (4 waves, two query elements, 4 per workgroup)",
     _SW.resized(batch=16, heads=3, grid_h=80, grid_w=80, window=10), [0, 15], [0, 2], [0, 1, 2, 3, 4, 63]),
]


@pytest.mark.parametrize("label,w,bs,hs,units", MULTI_UNIT)
def test_multi_unit_workgroups(dev, label, w, bs, hs, units):
    w = fit(w) if w.mode != "none" else w
    say("multi-unit", label, w.qkv_shape)
    compare(w, make_inputs(w, sigma=1.0, seed=9000), dev, batch_sel=bs, heads_sel=hs, units=units)


FULL_SAMPLES = {
    # workload: (batch indices, head indices) checked against the oracle
    "swin_tiny": (None, None),
    "swin_t_w7": ([0, 31], [0, 2]),
    "deit_s_irpe_k": ([0, 37, 63], [0, 5]),
    "deit_s_irpe_qkv": ([0, 63], [1, 4]),
    "highres_irpe_k": ([3], [5]),
    "deit_s_irpe_bias": ([0, 63], [0, 5]),
    "deit_s_irpe_k_cross": ([0, 63], [2]),
    "detr_irpe_k": ([0, 7], [0, 7]),
    "deit_s_irpe_bias_euclid": ([0, 63], [0, 5]),
    "detr_wide_irpe_k": ([1], [7]),
    "swin_t_w7_irpe_qkv": ([0, 31], [0, 2]),
}


def test_full_size_highres_sigma1(dev):
    # The 56 x 56 grid at full size with sigma = 1 tables, one (batch, head)
    # checked against the oracle: offsets up to 55 reach the outermost row and
    # column buckets (index 8 of 17, |offset| >= 29) at a scale where the key
    # term moves the output far more than the tolerance.
    w = WORKLOADS["highres_irpe_k"]
    say("full size sigma 1", w.qkv_shape, "sampled (b, h): [1], [3]")
    compare(w, make_inputs(w, sigma=1.0), dev, batch_sel=[1], heads_sel=[3])


@pytest.mark.parametrize("name", list(FULL_SAMPLES))
def test_full_size_sampled(dev, name):
    w = WORKLOADS[name]
    bs, hs = FULL_SAMPLES[name]
    say("full size", name, w.qkv_shape, "sampled (b, h):", bs, hs)
    x = make_inputs(w)
    units = None
    if name == "swin_t_w7":
        units = [0, 9, 27, 63]
    compare(w, x, dev, batch_sel=bs, heads_sel=hs, units=units)
