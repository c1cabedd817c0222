"""The allocation-free backward (rpe_attn_bwd_noalloc, through the C ABI) against
rpe_attn_bwd with a caller workspace: two calls in a row, the second on a smaller
problem, and a problem whose workspace exceeds the library's array (refused
before any launch).  Both entry points run the same kernels; where the table
gradients are summed in a fixed order the results are bit-identical, and every
gradient is also held to the oracle backward's tolerance."""

import numpy as np
import pytest

from oracle import Spec, num_buckets
from oracle.backward import attention_backward
from vision_transformer_attention_amd.workloads import WORKLOADS, make_inputs, round_to_dtype

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
                alpha=w.alpha, beta=w.beta, gamma=w.gamma, reading=w.reading, tables_per_head=w.tables_per_head)


def _fit(w):
    return w.resized(table_rows=num_buckets(_spec(w))[2]) if w.mode != "none" else w


def _run(dev, w, seed):
    import torch
    import vision_transformer_attention_amd as pkg
    x = make_inputs(w, sigma=1.0, seed=seed)
    dout = round_to_dtype(np.random.default_rng(seed + 1).standard_normal(w.qkv_shape), w.dtype)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t = {n: torch.from_numpy(np.ascontiguousarray(a)).to(torch.float32 if n == "bias" else tdt).to(dev)
         for n, a in x.items()}
    td = torch.from_numpy(dout).to(tdt).to(dev)
    kw = dict(grid=(w.grid_h, w.grid_w), window=w.window, prefix_tokens=w.prefix, mode=w.mode,
              terms="".join(sorted(w.terms)), map=w.map, alpha=w.alpha, beta=w.beta, gamma=w.gamma,
              rounding=w.reading, bias=t.get("bias"), rq=t.get("rq"), rk=t.get("rk"), rv=t.get("rv"))
    _, lse = pkg.rpe_attn_fwd(t["q"], t["k"], t["v"], return_lse=True, **kw)
    g_ws = pkg.rpe_attn_bwd(t["q"], t["k"], t["v"], td, lse, **kw)
    g_na = pkg.rpe_attn_bwd_noalloc(t["q"], t["k"], t["v"], td, lse, **kw)
    torch.cuda.synchronize()
    return x, dout, g_ws, g_na


_D = WORKLOADS["deit_s_irpe_k"]
# (label, larger problem, smaller problem run right after it)
PAIRS = [
    ("contextual KV bf16 d64: 14x14 + cls then 7x9 + cls",
     _D.resized(batch=2, heads=3, terms=frozenset("kv")),
     _D.resized(batch=1, heads=2, grid_h=7, grid_w=9, terms=frozenset("kv"))),
    ("bias, Swin 7x7 windows then one window",
     WORKLOADS["swin_t_w7"].resized(batch=2, heads=3, grid_h=14, grid_w=21),
     WORKLOADS["swin_t_w7"].resized(batch=1, heads=3, grid_h=7, grid_w=7)),
    ("contextual KQV fp32: 9x9 + cls then 5x6 + cls",
     _D.resized(batch=2, heads=2, head_dim=32, grid_h=9, grid_w=9, terms=frozenset("kqv"), dtype="fp32"),
     _D.resized(batch=1, heads=2, head_dim=32, grid_h=5, grid_w=6, terms=frozenset("kqv"), dtype="fp32")),
]


@pytest.mark.parametrize("label,big,small", PAIRS)
def test_noalloc_matches_workspace_entry(dev, label, big, small):
    for w in (_fit(big), _fit(small)):
        print("[case] bwd noalloc", label, w.qkv_shape, flush=True)
        x, dout, g_ws, g_na = _run(dev, w, 9970)
        ref = attention_backward(_spec(w), x["q"], x["k"], x["v"], dout, bias=x.get("bias"), rq=x.get("rq"),
                                 rk=x.get("rk"), rv=x.get("rv"))
        assert set(g_na) == set(g_ws)
        # the table gradients are summed in a fixed order when the per-unit partial sums
        # fit the workspace's weight region, else with float atomics (order may vary)
        units = w.batch * w.heads * (((w.grid_h // w.window) * (w.grid_w // w.window)) if w.window else 1)
        t = w.prefix + ((w.window * w.window) if w.window else w.grid_h * w.grid_w)
        kinds = len(w.terms) if w.mode == "contextual" else 0
        fixed_order = units * w.table_rows * (kinds * w.head_dim + (1 if w.mode == "bias" else 0)) <= units * t * t
        for n in sorted(g_ws):
            a = g_na[n].cpu().numpy().astype(np.float64)
            b = g_ws[n].cpu().numpy().astype(np.float64)
            scale = max(1.0, float(np.abs(ref[n]).max()))
            err = float(np.abs(a - ref[n]).max())
            print(f"    {n}: noalloc vs workspace max diff {float(np.abs(a - b).max()):.3e}; "
                  f"vs oracle {err:.3e} (rel tol {REL[w.dtype]} x {scale:.3e})", flush=True)
            if n in ("dq", "dk", "dv") or fixed_order:
                assert np.array_equal(a, b), n
            else:
                assert float(np.abs(a - b).max()) <= 1e-5 * scale, n
            assert np.isfinite(a).all() and err <= REL[w.dtype] * scale, (n, err)


def test_noalloc_refuses_large_workspace(dev):
    import ctypes
    import torch
    import vision_transformer_attention_amd as pkg
    from vision_transformer_attention_amd import _lib
    # DeiT-S iRPE-K at full batch needs about 120 MB of workspace, above the array
    w = WORKLOADS["deit_s_irpe_k"]
    d = pkg.make_desc(batch=w.batch, heads=w.heads, head_dim=w.head_dim, grid=(w.grid_h, w.grid_w),
                      prefix_tokens=w.prefix, mode="contextual", terms="k", map="piecewise", alpha=w.alpha,
                      beta=w.beta, gamma=w.gamma)
    n = ctypes.c_uint64()
    assert pkg.load().rpe_attn_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0
    assert n.value > _lib.BWD_NOALLOC_MAX_BYTES
    one = ctypes.c_void_p(256)
    print("[case] bwd noalloc refuses", n.value, "bytes", flush=True)
    st = pkg.load().rpe_attn_bwd_noalloc(ctypes.byref(d), *([one] * 16), None)
    assert st == -2
    torch.cuda.synchronize()
