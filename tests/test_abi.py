"""C-ABI library on the CPU: it loads, exports every declared symbol, and its
validation and size queries agree with the oracle.  No compute call is made
(none of these entry points touches the device)."""

import ctypes
import os
import re
import shutil
import subprocess

import pytest

import vision_transformer_attention_amd as pkg
from vision_transformer_attention_amd import _lib
from vision_transformer_attention_amd.workloads import WORKLOADS

from oracle import Spec, num_buckets

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib_or_skip():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("librpe_attn.so not built (run __graft_entry__.build())")
    return pkg.load()


def test_exports_every_declared_symbol():
    lib = _lib_or_skip()
    header = open(os.path.join(ROOT, "include", "rpe_attn.h")).read()
    declared = set(re.findall(r"^(?:rpe_status|const char\*)\s+(rpe_\w+)\s*\(", header, re.M))
    assert declared == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
        for name in declared:
            assert re.search(rf"\bT {name}\b", out), name
    assert lib.rpe_attn_version().decode().startswith("rpe_attn")


def test_roof_probes_export_their_header():
    path = os.path.join(ROOT, "vision_transformer_attention_amd", "librpe_roofs.so")
    if not os.path.exists(path):
        pytest.skip("librpe_roofs.so not built (run __graft_entry__.build())")
    header = open(os.path.join(ROOT, "include", "rpe_roofs.h")).read()
    declared = set(re.findall(r"^int32_t\s+(rpe_roof_\w+)\s*\(", header, re.M))
    assert declared == {"rpe_roof_copy", "rpe_roof_read", "rpe_roof_mfma_bf16", "rpe_roof_fma_f32",
                        "rpe_roof_exp2_f32"}
    lib = ctypes.CDLL(path)
    for name in declared:
        assert hasattr(lib, name), name
    # argument checks return before any device call
    work = ctypes.c_double(0.0)
    f = lib.rpe_roof_copy
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)]
    f.restype = ctypes.c_int32
    assert f(None, None, 16, None, ctypes.byref(work)) == -1
    assert f(1, 1, 15, None, ctypes.byref(work)) == -1
    r = lib.rpe_roof_read
    r.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.POINTER(ctypes.c_double)]
    r.restype = ctypes.c_int32
    assert r(1, 16, 0, 1, None, ctypes.byref(work)) == -1
    g = lib.rpe_roof_mfma_bf16
    g.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)]
    g.restype = ctypes.c_int32
    assert g(0, 1, None, ctypes.byref(work)) == -1


def _w_desc(w, **over):
    kw = dict(batch=w.batch, heads=w.heads, head_dim=w.head_dim, grid=(w.grid_h, w.grid_w),
              window=w.window, prefix_tokens=w.prefix, dtype=w.dtype, mode=w.mode,
              terms="".join(sorted(w.terms)), map=w.map, alpha=w.alpha, beta=w.beta, gamma=w.gamma,
              rounding=w.reading, tables_per_head=w.tables_per_head, method=w.method)
    kw.update(over)
    return pkg.make_desc(**kw)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_geometry_matches_oracle(name):
    _lib_or_skip()
    w = WORKLOADS[name]
    d = _w_desc(w)
    assert pkg.rpe_attn_validate(d) == 0
    spec = Spec(w.grid_h, w.grid_w, window=w.window, prefix=w.prefix, mode=w.mode, terms=w.terms,
                map=w.map, alpha=w.alpha, beta=w.beta, gamma=w.gamma, reading=w.reading, method=w.method)
    h, s, rows = pkg.rpe_attn_num_buckets(d)        # table rows: S*S, or 2S under Cross
    assert num_buckets(spec) == (h, s, rows)
    assert num_buckets(spec)[2] == w.table_rows
    n, t, u = pkg.rpe_attn_unit_size(d)
    assert (n, t, u) == (spec.tokens_per_image, spec.unit_tokens, spec.units_per_image)


@pytest.mark.parametrize("reading,beta,per_axis", [("capped", 3.8, 9), ("trunc", 3.8, 7),
                                                   ("capped", 7.6, 17), ("trunc", 7.6, 15),
                                                   ("capped", 3.5, 9), ("trunc", 3.5, 7)])
def test_half_width_readings(reading, beta, per_axis):
    _lib_or_skip()
    d = pkg.make_desc(grid=(14, 14), mode="contextual", terms="k", map="piecewise", alpha=1.0,
                      beta=beta, gamma=4 * beta, rounding=reading)
    assert pkg.rpe_attn_num_buckets(d)[1] == per_axis


BAD = [
    (dict(batch=-1), -2), (dict(heads=0), -2), (dict(grid=(0, 4)), -2), (dict(grid=(2000, 4)), -2),
    (dict(window=3, grid=(8, 8)), -2), (dict(window=4, grid=(8, 8), prefix_tokens=1), -2),
    (dict(prefix_tokens=17), -2), (dict(dtype=7), -3), (dict(mode=9), -4),
    (dict(mode="bias", map="swin", terms="v"), -5), (dict(mode="bias", terms="k"), -4),
    (dict(mode="contextual", terms=""), -4), (dict(mode="none", terms="k"), -4),
    (dict(mode="contextual", terms="k", map="piecewise", alpha=0.0, beta=2.0, gamma=8.0), -7),
    (dict(mode="contextual", terms="k", map="piecewise", alpha=2.0, beta=1.0, gamma=8.0), -7),
    (dict(mode="contextual", terms="k", map="piecewise", alpha=2.0, beta=3.0, gamma=2.0), -7),
    (dict(mode="contextual", terms="k", map="piecewise", alpha=2.0, beta=3.0, gamma=8.0, rounding=5), -4),
    (dict(head_dim=48), -8), (dict(head_dim=128), -8), (dict(scale=float("nan")), -7),
    (dict(grid=(4, 257)), -8),
]


@pytest.mark.parametrize("over,code", BAD)
def test_validation_codes(over, code):
    lib = _lib_or_skip()
    base = dict(batch=2, heads=2, head_dim=32, grid=(8, 8), dtype="bf16", mode="none")
    base.update(over)
    d = pkg.make_desc(**base)
    st = pkg.rpe_attn_validate(d)
    if code == -8 and st == 0:
        # unsupported configurations may pass validation and be refused by the planner:
        # rpe_attn_fwd must refuse them before touching the device
        st = lib.rpe_attn_fwd(ctypes.byref(d), *([ctypes.c_void_p(16)] * 4), None, None, None, None,
                              ctypes.c_void_p(16), None, None)
    assert st == code, (over, st, lib.rpe_status_str(st))


def test_fwd_rejects_before_device():
    lib = _lib_or_skip()
    one = ctypes.c_void_p(16)
    d = pkg.make_desc(batch=1, heads=1, head_dim=32, grid=(7, 7), window=7, mode="bias", map="swin")
    # bias table missing
    assert lib.rpe_attn_fwd(ctypes.byref(d), one, one, one, None, None, None, None, one, None, None) == -1
    # output missing
    assert lib.rpe_attn_fwd(ctypes.byref(d), one, one, one, one, None, None, None, None, None, None) == -1
    d = pkg.make_desc(batch=1, heads=1, head_dim=64, grid=(14, 14), prefix_tokens=1, mode="contextual",
                      terms="kv", map="piecewise", alpha=1.9, beta=3.8, gamma=15.2)
    assert lib.rpe_attn_fwd(ctypes.byref(d), one, one, one, None, None, one, None, one, None, None) == -1
    assert lib.rpe_attn_fwd(None, one, one, one, None, None, None, None, one, None, None) == -1
    assert lib.rpe_attn_bucket_map(ctypes.byref(d), None, None) == -1
    assert lib.rpe_attn_axis_index(ctypes.byref(d), 0, one, None) == -2
    assert lib.rpe_status_str(-5).decode().startswith("the value term")


def test_host_plan_fuzz_sanitized(tmp_path):
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("g++ missing")
    exe = str(tmp_path / "plan_fuzz")
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                    os.path.join(ROOT, "tests", "host", "plan_fuzz.cpp"),
                    os.path.join(ROOT, "vision_transformer_attention_amd", "csrc", "plan.cpp"), "-o", exe],
                   check=True)
    r = subprocess.run([exe, "40000"], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout


def test_cross_to_product_rejects_before_device():
    lib = _lib_or_skip()
    one = ctypes.c_void_p(16)
    B, V = _lib.RPE_TABLE_BIAS, _lib.RPE_TABLE_VECTOR
    ctx = pkg.make_desc(batch=1, heads=2, head_dim=64, grid=(14, 14), prefix_tokens=1, mode="contextual",
                        terms="k", map="piecewise", alpha=1.9, beta=3.8, gamma=15.2)
    bias = pkg.make_desc(batch=1, heads=2, head_dim=32, grid=(7, 7), window=7, mode="bias", map="swin")
    none = pkg.make_desc(batch=1, heads=2, head_dim=32, grid=(7, 7), mode="none")
    f = lib.rpe_attn_cross_to_product
    assert f(None, V, one, one, None) == -1
    assert f(ctypes.byref(ctx), V, None, one, None) == -1
    assert f(ctypes.byref(ctx), V, one, None, None) == -1
    # a kind the mode has no table for, an unknown kind, no position mode
    assert f(ctypes.byref(ctx), B, one, one, None) == -4
    assert f(ctypes.byref(bias), V, one, one, None) == -4
    assert f(ctypes.byref(ctx), 7, one, one, None) == -4
    assert f(ctypes.byref(none), B, one, one, None) == -4
    # descriptor validation comes first
    bad = pkg.make_desc(batch=1, heads=2, head_dim=64, grid=(14, 14), mode="contextual", terms="k",
                        map="piecewise", alpha=-1.0, beta=3.8, gamma=15.2)
    assert f(ctypes.byref(bad), V, one, one, None) == -7


@pytest.mark.parametrize("m", ["euclidean", "euclidean_rounded", "quantized", "quantized_squared"])
def test_undirected_maps_geometry_and_rejections(m):
    lib = _lib_or_skip()
    one = ctypes.c_void_p(16)
    d = pkg.make_desc(batch=1, heads=2, head_dim=64, grid=(14, 14), prefix_tokens=1, mode="contextual",
                      terms="k", map=m, alpha=1.9, beta=3.8, gamma=15.2)
    assert pkg.rpe_attn_validate(d) == 0
    spec = Spec(14, 14, prefix=1, mode="contextual", terms={"k"}, map=m, alpha=1.9, beta=3.8, gamma=15.2)
    assert pkg.rpe_attn_num_buckets(d) == num_buckets(spec) == (4, 9, 9)
    # the per-axis tools have no undirected form; the forward, the pair map (rows
    # u + H) and the backward take the undirected tables as they are
    assert lib.rpe_attn_fwd(ctypes.byref(d), None, one, one, None, None, one, None, one, None, None) == -1
    assert lib.rpe_attn_bucket_map(ctypes.byref(d), None, None) == -1
    assert lib.rpe_attn_axis_index(ctypes.byref(d), 5, one, None) == -4
    n = ctypes.c_uint64()
    assert lib.rpe_attn_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0
    assert lib.rpe_attn_cross_to_product(ctypes.byref(d), _lib.RPE_TABLE_VECTOR, one, one, None) == -4
    f = lib.rpe_attn_undirected_to_product
    assert f(ctypes.byref(d), _lib.RPE_TABLE_VECTOR, None, one, None) == -1
    assert f(ctypes.byref(d), _lib.RPE_TABLE_BIAS, one, one, None) == -4
    big = pkg.make_desc(batch=1, heads=2, head_dim=64, grid=(100, 100), mode="bias", map=m,
                        alpha=1.9, beta=3.8, gamma=15.2)
    assert f(ctypes.byref(big), _lib.RPE_TABLE_BIAS, one, one, None) == -6     # 199^2 raw offsets
    assert lib.rpe_attn_bucket_map(ctypes.byref(big), one, None) == -6
    assert lib.rpe_attn_bwd_workspace_size(ctypes.byref(big), ctypes.byref(n)) == -6
    # the bound is on the squared offset lengths, (R-1)^2 + (C-1)^2 < 16384: a
    # 2 x 127 grid (126^2 + 1) is taken, a 2 x 129 grid is not
    for gw, want in ((127, 0), (129, -6)):
        wide = pkg.make_desc(batch=1, heads=2, head_dim=64, grid=(2, gw), mode="bias", map=m,
                             alpha=1.9, beta=3.8, gamma=15.2)
        assert lib.rpe_attn_bwd_workspace_size(ctypes.byref(wide), ctypes.byref(n)) == want
        assert lib.rpe_attn_bucket_map(ctypes.byref(wide), None, None) == (-1 if want == 0 else want)
    pw = pkg.make_desc(batch=1, heads=2, head_dim=64, grid=(14, 14), mode="bias", map="piecewise",
                       alpha=1.9, beta=3.8, gamma=15.2)
    assert f(ctypes.byref(pw), _lib.RPE_TABLE_BIAS, one, one, None) == -4       # not undirected


def test_bwd_rejects_before_device():
    lib = _lib_or_skip()
    one = ctypes.c_void_p(16)
    d = pkg.make_desc(batch=1, heads=2, head_dim=64, grid=(14, 14), prefix_tokens=1, mode="contextual",
                      terms="kv", map="piecewise", alpha=1.9, beta=3.8, gamma=15.2)
    n = ctypes.c_uint64()
    assert lib.rpe_attn_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0
    T = 197
    # bucket map + P + dL of 2 units (rows padded to 224 floats), then the K and V bucket sums
    # (81 per row), each 256-B aligned
    up = lambda v: (v + 255) // 256 * 256
    Ts = 224
    assert n.value == up(T * T * 2) + 2 * up(2 * T * Ts * 4) + 2 * up(2 * T * 81 * 4)
    assert lib.rpe_attn_bwd_workspace_size(ctypes.byref(d), None) == -1
    args = [one] * 16
    # the value table's gradient missing (rv given, drv NULL)
    a = list(args)
    a[15] = None
    assert lib.rpe_attn_bwd(ctypes.byref(d), *a, one, ctypes.c_uint64(n.value), None) == -1
    # workspace too small
    assert lib.rpe_attn_bwd(ctypes.byref(d), *args, one, ctypes.c_uint64(n.value - 1), None) == -2
    assert lib.rpe_attn_bwd(None, *args, one, ctypes.c_uint64(n.value), None) == -1


def test_descriptor_layout():
    # the ctypes mirror matches the C struct: 12 int32 fields, three doubles, the
    # scale, tables_per_head, method, then seven int64 fields (8-byte aligned)
    assert ctypes.sizeof(_lib.Desc) == 48 + 24 + 4 + 4 + 4 + 4 + 7 * 8
    assert _lib.Desc.table_head_stride.offset == 88 and _lib.Desc.o_stride_n.offset == 136


STRIDE_BAD = [
    # (strides, o_strides, code): all-zero or all-positive, stride_n >= head_dim, 16-byte rows
    ((1, 0, 0), None, -2), ((0, 0, 32), None, -2), ((6000, 200, 16), None, -2),
    ((6000, 200, 36), None, -10), (None, (6000, 200, 36), -10), ((6004, 200, 32), None, -10),
    ((1 << 40, 32, 1 << 30), None, -2),
]


@pytest.mark.parametrize("strides,o_strides,code", STRIDE_BAD)
def test_stride_validation(strides, o_strides, code):
    _lib_or_skip()
    d = pkg.make_desc(batch=2, heads=2, head_dim=32, grid=(8, 8), dtype="bf16", mode="none",
                      strides=strides, o_strides=o_strides)
    assert pkg.rpe_attn_validate(d) == code


def test_stride_views_accepted():
    _lib_or_skip()
    B, N, H, d = 2, 65, 3, 64
    # q, k, v as slices of a fused [B][N][3][H][d] projection, o as [B][N][H][d]
    fused = dict(strides=(N * 3 * H * d, d, 3 * H * d), o_strides=(N * H * d, d, H * d))
    desc = pkg.make_desc(batch=B, heads=H, head_dim=d, grid=(8, 8), prefix_tokens=1, mode="contextual",
                         terms="k", map="piecewise", alpha=1.9, beta=3.8, gamma=15.2, **fused)
    assert pkg.rpe_attn_validate(desc) == 0


def test_method_validation_and_geometry():
    lib = _lib_or_skip()
    one = ctypes.c_void_p(16)
    kw = dict(batch=1, heads=2, head_dim=64, grid=(14, 14), prefix_tokens=1, alpha=1.9, beta=3.8, gamma=15.2)
    cross = pkg.make_desc(mode="contextual", terms="k", map="piecewise", method="cross", **kw)
    assert pkg.rpe_attn_validate(cross) == 0
    assert pkg.rpe_attn_num_buckets(cross) == (4, 9, 18)
    # the Cross mapping needs a table and a directed map
    assert pkg.rpe_attn_validate(pkg.make_desc(mode="none", method="cross", **kw)) == -4
    assert pkg.rpe_attn_validate(pkg.make_desc(mode="bias", map="euclidean", method="cross", **kw)) == -4
    assert pkg.rpe_attn_validate(pkg.make_desc(mode="bias", map="piecewise", method=2, **kw)) == -4
    # the backward takes either method, and contiguous tensors only; under Cross
    # its workspace holds a second pair-to-row map ([T][T] int16, 256-byte aligned)
    n = ctypes.c_uint64()
    assert lib.rpe_attn_bwd_workspace_size(ctypes.byref(cross), ctypes.byref(n)) == 0
    m = ctypes.c_uint64()
    prod = pkg.make_desc(mode="contextual", terms="k", map="piecewise", **kw)
    assert lib.rpe_attn_bwd_workspace_size(ctypes.byref(prod), ctypes.byref(m)) == 0
    t = 197
    rows_bytes = lambda rows: (2 * t * rows * 4 + 255) // 256 * 256     # B H U T rows floats
    assert n.value - m.value == (t * t * 2 + 255) // 256 * 256 + rows_bytes(18) - rows_bytes(81)
    strided = pkg.make_desc(mode="contextual", terms="k", map="piecewise",
                            strides=(197 * 3 * 2 * 64, 64, 3 * 2 * 64), **kw)
    assert lib.rpe_attn_bwd_workspace_size(ctypes.byref(strided), ctypes.byref(n)) == -8
    # misaligned pointers and too-small table head strides are refused before any launch
    d = pkg.make_desc(mode="contextual", terms="k", map="piecewise", **kw)
    odd = ctypes.c_void_p(18)
    assert lib.rpe_attn_fwd(ctypes.byref(d), odd, one, one, None, None, one, None, one, None, None) == -10
    assert lib.rpe_attn_fwd(ctypes.byref(d), one, one, one, None, None, odd, None, one, None, None) == -10
    ph = pkg.make_desc(mode="contextual", terms="k", map="piecewise", tables_per_head=True,
                       table_head_stride=81 * 64 - 8, **kw)
    assert lib.rpe_attn_fwd(ctypes.byref(ph), one, one, one, None, None, one, None, one, None, None) == -2
    assert lib.rpe_status_str(-10).decode().startswith("a pointer or stride")


def _plan(**kw):
    base = dict(batch=2, heads=2, head_dim=64, grid=(14, 14), mode="contextual", terms="k", map="piecewise",
                alpha=1.9, beta=3.8, gamma=15.2)
    base.update(kw)
    return pkg.rpe_attn_fwd_plan(pkg.make_desc(**base))


def test_fwd_plan_row_slots_and_blocks():
    _lib_or_skip()
    # rows padded to the power of two up to 64 slots, to a multiple of 32 beyond
    for (gh, gw), slots in (((14, 14), 16), ((56, 56), 64), ((50, 84), 96), ((3, 200), 224), ((2, 256), 256),
                            ((7, 65), 96)):
        p = _plan(grid=(gh, gw))
        assert p["row_slots"] == slots, (gw, p)
        assert p["key_blocks"] == (gh * slots + 31) // 32   # no prefix tokens
    # a class token in the row padding adds no block; with no padding left it takes a block of its own
    assert _plan(grid=(14, 14), prefix_tokens=1)["key_blocks"] == 7
    assert _plan(grid=(2, 96), prefix_tokens=1)["key_blocks"] == 2 * 3 + 1


def test_fwd_plan_fits_and_counts():
    _lib_or_skip()
    for kw in (dict(), dict(terms="kqv"), dict(terms="kqv", dtype="fp32", head_dim=32),
               dict(mode="bias", terms="", grid=(56, 56), window=7, map="swin", tables_per_head=True),
               dict(grid=(50, 84), head_dim=32), dict(mode="none", terms="", map="swin", grid=(4, 150))):
        p = _plan(**kw)
        assert 0 < p["lds_bytes"] <= 160 * 1024
        assert 2 <= p["waves_per_group"] <= 4 and p["waves_per_simd"] in (2, 3, 4)
        units = 2 * 2 * ((kw.get("grid", (14, 14))[0] // kw["window"]) ** 2 if kw.get("window") else 1)
        assert p["workgroups"] * p["units_per_group"] == units * p["query_chunks"]
    assert _plan()["value_term"] == "none"
    assert _plan(terms="kqv")["value_term"] == "per key block"
    assert _plan(terms="v", dtype="fp32", head_dim=32)["value_term"] in ("per (row bucket, key column) sums",
                                                                          "per-bucket sums")


def test_fwd_plan_errors():
    lib = _lib_or_skip()
    d = pkg.make_desc(batch=1, heads=1, head_dim=64, grid=(14, 14), mode="none")
    assert lib.rpe_attn_fwd_plan(ctypes.byref(d), None) == -1
    wide = pkg.make_desc(batch=1, heads=1, head_dim=64, grid=(2, 257), mode="none")
    with pytest.raises(pkg.RpeError):
        pkg.rpe_attn_fwd_plan(wide)
