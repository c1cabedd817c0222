"""Python binding of librpe_attn (argument marshalling only).

Names mirror the C entry points of include/rpe_attn.h.  PyTorch provides the
device memory and the current HIP stream; every step of the computation runs
in the library's kernels.  There is no fallback path: a missing library or a
rejected call raises.
"""

import ctypes

from . import _lib
from ._lib import Desc, check, load

_MODES = {"none": _lib.RPE_MODE_NONE, "bias": _lib.RPE_MODE_BIAS,
          "contextual": _lib.RPE_MODE_CONTEXTUAL}
_MAPS = {"swin": _lib.RPE_MAP_SWIN, "piecewise": _lib.RPE_MAP_PIECEWISE, "euclidean": _lib.RPE_MAP_EUCLIDEAN,
         "euclidean_rounded": _lib.RPE_MAP_EUCLIDEAN_ROUNDED, "quantized": _lib.RPE_MAP_QUANTIZED,
         "quantized_squared": _lib.RPE_MAP_QUANTIZED_SQUARED}
UNDIRECTED = ("euclidean", "euclidean_rounded", "quantized", "quantized_squared")
_ROUNDING = {"capped": _lib.RPE_ROUND_CAPPED, "trunc": _lib.RPE_ROUND_TRUNC}
_TERM_BITS = {"k": _lib.RPE_TERM_K, "q": _lib.RPE_TERM_Q, "v": _lib.RPE_TERM_V}


def _torch():
    import torch
    return torch


_METHODS = {"product": _lib.RPE_METHOD_PRODUCT, "cross": _lib.RPE_METHOD_CROSS}


def make_desc(*, batch=1, heads=1, head_dim=64, grid=(1, 1), window=0, prefix_tokens=0,
              dtype="bf16", mode="none", terms="", map="swin", alpha=0.0, beta=0.0, gamma=0.0,
              rounding="capped", scale=None, tables_per_head=False, method="product",
              strides=None, o_strides=None, table_head_stride=0):
    """Build an ``rpe_attn_desc``.  ``terms`` is a string or set over 'k', 'q', 'v';
    ``strides`` / ``o_strides`` are the (batch, head, token) element strides of
    q, k, v and of o (None: contiguous)."""
    d = Desc()
    d.batch, d.heads, d.head_dim = int(batch), int(heads), int(head_dim)
    d.grid_h, d.grid_w = int(grid[0]), int(grid[1])
    d.window, d.prefix_tokens = int(window), int(prefix_tokens)
    d.dtype = {"bf16": _lib.RPE_BF16, "fp32": _lib.RPE_FP32}[dtype] if isinstance(dtype, str) else int(dtype)
    d.mode = _MODES[mode] if isinstance(mode, str) else int(mode)
    bits = 0
    for t in terms:
        bits |= _TERM_BITS[t]
    d.terms = bits
    d.map = _MAPS[map] if isinstance(map, str) else int(map)
    d.rounding = _ROUNDING[rounding] if isinstance(rounding, str) else int(rounding)
    d.alpha, d.beta, d.gamma = float(alpha), float(beta), float(gamma)
    d.scale = 0.0 if scale is None else float(scale)
    d.tables_per_head = 1 if tables_per_head else 0
    d.method = _METHODS[method] if isinstance(method, str) else int(method)
    d.table_head_stride = int(table_head_stride)
    d.stride_b, d.stride_h, d.stride_n = (0, 0, 0) if strides is None else (int(x) for x in strides)
    d.o_stride_b, d.o_stride_h, d.o_stride_n = (0, 0, 0) if o_strides is None else (int(x) for x in o_strides)
    return d


def rpe_attn_validate(desc):
    return load().rpe_attn_validate(ctypes.byref(desc))


def rpe_attn_num_buckets(desc):
    """(half_width, per_axis, total) of the bucket table."""
    h, s, t = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    check("rpe_attn_num_buckets",
          load().rpe_attn_num_buckets(ctypes.byref(desc), ctypes.byref(h), ctypes.byref(s), ctypes.byref(t)))
    return h.value, s.value, t.value


def rpe_attn_unit_size(desc):
    """(tokens per image N, tokens per unit T, units per image)."""
    n, t, u = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    check("rpe_attn_unit_size",
          load().rpe_attn_unit_size(ctypes.byref(desc), ctypes.byref(n), ctypes.byref(t), ctypes.byref(u)))
    return n.value, t.value, u.value


_VALUE_TERM = {0: "none", 1: "per key block", 2: "per (row bucket, key column) sums", 3: "per-bucket sums"}


def rpe_attn_fwd_plan(desc):
    """The launch plan rpe_attn_fwd makes for ``desc`` (host only), as a dict."""
    from ._lib import PlanInfo
    info = PlanInfo()
    check("rpe_attn_fwd_plan", load().rpe_attn_fwd_plan(ctypes.byref(desc), ctypes.byref(info)))
    out = {name: getattr(info, name) for name, _ in PlanInfo._fields_ if name != "reserved"}
    out["value_term"] = _VALUE_TERM[out["value_term"]]
    return out


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def rpe_attn_axis_index(desc, length, device="cuda"):
    """g(x) for x = -(length-1) .. length-1 as an int16 device tensor."""
    torch = _torch()
    out = torch.empty(2 * length - 1, dtype=torch.int16, device=device)
    check("rpe_attn_axis_index",
          load().rpe_attn_axis_index(ctypes.byref(desc), int(length), ctypes.c_void_p(out.data_ptr()),
                                     _stream(out.device)))
    return out


def rpe_attn_bucket_map(desc, device="cuda"):
    """[T, T] int16 bucket ids of one unit (-1 where a prefix token takes part)."""
    torch = _torch()
    _, t, _ = rpe_attn_unit_size(desc)
    out = torch.empty((t, t), dtype=torch.int16, device=device)
    check("rpe_attn_bucket_map",
          load().rpe_attn_bucket_map(ctypes.byref(desc), ctypes.c_void_p(out.data_ptr()),
                                     _stream(out.device)))
    return out


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def rpe_attn_cross_to_product(desc, table):
    """The Product table [T, S*S(, d)] equal to a Cross table [T, 2S(, d)]
    (rows [0, S): row-offset encodings, [S, 2S): column-offset encodings).
    A 2-D float32 table is a bias table, a 3-D one a contextual table."""
    torch = _torch()
    _, s, _ = rpe_attn_num_buckets(desc)
    nb = s * s
    kind = _lib.RPE_TABLE_BIAS if table.dim() == 2 else _lib.RPE_TABLE_VECTOR
    th = desc.heads if desc.tables_per_head else 1
    want = (th, 2 * s) if kind == _lib.RPE_TABLE_BIAS else (th, 2 * s, desc.head_dim)
    if tuple(table.shape) != want or not table.is_contiguous() or not table.is_cuda:
        raise ValueError(f"cross table must be a contiguous device tensor {list(want)}")
    out = torch.empty((th, nb) + tuple(table.shape[2:]), dtype=table.dtype, device=table.device)
    check("rpe_attn_cross_to_product",
          load().rpe_attn_cross_to_product(ctypes.byref(desc), int(kind), _ptr(table), _ptr(out),
                                           _stream(table.device)))
    return out


def rpe_attn_undirected_to_product(desc, table):
    """The Swin-map table over raw offsets [T, S'*S'(, d)] equal to an undirected-map
    table [T, S(, d)] (S from rpe_attn_num_buckets, S' = 2 max(R, C) - 1)."""
    torch = _torch()
    _, s, rows = rpe_attn_num_buckets(desc)
    kind = _lib.RPE_TABLE_BIAS if table.dim() == 2 else _lib.RPE_TABLE_VECTOR
    th = desc.heads if desc.tables_per_head else 1
    want = (th, rows) if kind == _lib.RPE_TABLE_BIAS else (th, rows, desc.head_dim)
    if tuple(table.shape) != want or not table.is_contiguous() or not table.is_cuda:
        raise ValueError(f"undirected table must be a contiguous device tensor {list(want)}")
    r = desc.window if desc.window else desc.grid_h
    c = desc.window if desc.window else desc.grid_w
    sp = 2 * max(r, c) - 1
    out = torch.empty((th, sp * sp) + tuple(table.shape[2:]), dtype=table.dtype, device=table.device)
    check("rpe_attn_undirected_to_product",
          load().rpe_attn_undirected_to_product(ctypes.byref(desc), int(kind), _ptr(table), _ptr(out),
                                                _stream(table.device)))
    return out


def _check_geometry_and_tables(desc, q, mode, terms, per_head, bias, rq, rk, rv):
    """Checks shared by the forward and backward bindings, before any launch: the
    library sizes every read and write from the descriptor alone, so the token
    count must match the grid and each table the mode and terms use must have
    the descriptor's shape, dtype and device."""
    torch = _torch()
    B, H, N, d = q.shape
    n_img, _, _ = rpe_attn_unit_size(desc)
    if n_img != N:
        raise ValueError(f"N = {N} but prefix_tokens + grid gives {n_img}")
    use = {"bias": mode == "bias", "rq": mode == "contextual" and "q" in terms,
           "rk": mode == "contextual" and "k" in terms, "rv": mode == "contextual" and "v" in terms}
    if mode == "none":
        return
    _, _, nb = rpe_attn_num_buckets(desc)
    th = H if per_head else 1
    for name, t in (("bias", bias), ("rq", rq), ("rk", rk), ("rv", rv)):
        if not use[name]:
            continue
        if t is None:
            raise ValueError(f"{name} is required by mode {mode!r} and terms {terms!r}")
        if name == "bias":
            if t.dtype != torch.float32 or tuple(t.shape) != (th, nb) or not t.is_contiguous():
                raise ValueError(f"bias must be contiguous float32 [{th}, {nb}]")
        elif t.dtype != q.dtype or tuple(t.shape) != (th, nb, d) or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous {q.dtype} [{th}, {nb}, {d}]")
        if not t.is_cuda or t.device != q.device:
            raise ValueError(f"{name} must be on the device of q")


def _view_strides(t, name):
    """(batch, head, token) element strides of a [B, H, N, d] view whose head dim is contiguous."""
    if t.dim() != 4 or t.stride(-1) != 1:
        raise ValueError(f"{name} must be a [B, H, N, d] view with a contiguous last dimension")
    return tuple(int(x) for x in t.stride()[:3])


def _fwd_setup(q, k, v, out, *, grid, window=0, prefix_tokens=0, mode="none", terms="", map="swin",
               alpha=0.0, beta=0.0, gamma=0.0, rounding="capped", scale=None, bias=None, rq=None, rk=None,
               rv=None, method="product"):
    """Validate a forward call and marshal it: (descriptor, out, [bias, rq, rk, rv] as
    launched)."""
    torch = _torch()
    if method not in _METHODS:
        raise ValueError(f"method {method!r}")
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must be [B, H, N, d] of one shape")
    if not (q.is_cuda and k.is_cuda and v.is_cuda) or k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be tensors on one device")
    if q.dtype not in (torch.bfloat16, torch.float32) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must all be bfloat16 or all float32")
    strides = _view_strides(q, "q")
    if _view_strides(k, "k") != strides or _view_strides(v, "v") != strides:
        raise ValueError("q, k and v must share their strides (pass .contiguous() copies otherwise)")
    B, H, N, d = q.shape
    if out is None:
        out = torch.empty((B, H, N, d), dtype=q.dtype, device=q.device)
    elif out.shape != q.shape or out.dtype != q.dtype or out.device != q.device:
        raise ValueError("out must match q in shape, dtype and device")
    o_strides = _view_strides(out, "out")
    tabs = [t for t in (bias, rq, rk, rv) if t is not None]
    per_head = any(t.shape[0] == H and H > 1 for t in tabs)
    desc = make_desc(batch=B, heads=H, head_dim=d, grid=grid, window=window, prefix_tokens=prefix_tokens,
                     dtype="bf16" if q.dtype == torch.bfloat16 else "fp32", mode=mode, terms=terms, map=map,
                     alpha=alpha, beta=beta, gamma=gamma, rounding=rounding, scale=scale,
                     tables_per_head=per_head, method=method, strides=strides, o_strides=o_strides)
    if mode == "none" and method == "cross":
        raise ValueError("the Cross mapping needs bias or contextual mode")
    _check_geometry_and_tables(desc, q, mode, terms, per_head, bias, rq, rk, rv)
    used = {"bias": mode == "bias", "rq": mode == "contextual" and "q" in terms,
            "rk": mode == "contextual" and "k" in terms, "rv": mode == "contextual" and "v" in terms}
    launch = [t if used[n] else None for n, t in zip(("bias", "rq", "rk", "rv"), (bias, rq, rk, rv))]
    if map in UNDIRECTED and mode == "none":
        raise ValueError("an undirected map needs bias or contextual mode")
    return desc, out, launch


def rpe_attn_fwd(q, k, v, *, grid, window=0, prefix_tokens=0, mode="none", terms="", map="swin",
                 alpha=0.0, beta=0.0, gamma=0.0, rounding="capped", scale=None, bias=None,
                 rq=None, rk=None, rv=None, out=None, return_lse=False, method="product"):
    """Attention forward with 2D relative position terms.

    q, k, v: [B, H, N, d] device views (bfloat16 or float32) with a contiguous
    last dimension and one set of strides (e.g. the three slices of a fused
    [B, N, 3, H, d] projection, permuted), N = prefix_tokens + grid[0] * grid[1].
    bias: [H or 1, rows] float32; rq / rk / rv: [H or 1, rows, d] in the dtype
    of q, contiguous; rows = S*S (method "product") or 2S (method "cross": the
    row-offset half, then the column-offset half), or S for an undirected map
    ("euclidean", "euclidean_rounded", "quantized", "quantized_squared"; rows
    H .. 2H hold the indices 0 .. H).  ``out`` may be any
    [B, H, N, d] view with a contiguous last dimension (default: a new
    contiguous tensor).  Returns o (and the float32 log-sum-exp [B, H, N] with
    ``return_lse``).
    """
    torch = _torch()
    desc, out, launch = _fwd_setup(
        q, k, v, out, grid=grid, window=window, prefix_tokens=prefix_tokens, mode=mode, terms=terms, map=map,
        alpha=alpha, beta=beta, gamma=gamma, rounding=rounding, scale=scale, bias=bias, rq=rq, rk=rk, rv=rv,
        method=method)
    B, H, N, _ = q.shape
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if return_lse else None
    b, tq, tk, tv = launch
    check("rpe_attn_fwd",
          load().rpe_attn_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(b), _ptr(tq), _ptr(tk),
                              _ptr(tv), _ptr(out), _ptr(lse), _stream(q.device)))
    return (out, lse) if return_lse else out


class PreparedFwd:
    """A validated rpe_attn_fwd call with fixed tensors: each call() is one
    library call with pre-marshalled arguments (for launch loops and timing).

    The tensors passed to ``prepare_fwd`` must stay alive and keep their
    storage while this object is used.
    """

    def __init__(self, desc, ptrs, keep, device):
        self._lib = load()
        self._desc = desc
        self._args = ptrs
        self._keep = keep
        self._device = device

    def __call__(self, stream=None):
        torch = _torch()
        s = ctypes.c_void_p(torch.cuda.current_stream(self._device).cuda_stream if stream is None else stream)
        check("rpe_attn_fwd", self._lib.rpe_attn_fwd(ctypes.byref(self._desc), *self._args, s))


def prepare_fwd(q, k, v, *, out, lse=None, **kw):
    """Validate once (by running the call) and return a PreparedFwd for repeats."""
    rpe_attn_fwd(q, k, v, out=out, **kw)
    kw.pop("return_lse", None)
    desc, out, launch = _fwd_setup(q, k, v, out, **kw)
    ptrs = [_ptr(q), _ptr(k), _ptr(v)] + [_ptr(t) for t in launch] + [_ptr(out), _ptr(lse)]
    return PreparedFwd(desc, ptrs, (q, k, v, out, lse, launch), q.device)


class PreparedBwd:
    """A validated rpe_attn_bwd call with fixed tensors and workspace (for timing)."""

    def __init__(self, desc, args, keep, device):
        self._lib = load()
        self._desc = desc
        self._args = args
        self._keep = keep
        self._device = device

    def __call__(self, stream=None):
        torch = _torch()
        s = ctypes.c_void_p(torch.cuda.current_stream(self._device).cuda_stream if stream is None else stream)
        check("rpe_attn_bwd", self._lib.rpe_attn_bwd(ctypes.byref(self._desc), *self._args, s))


def prepare_bwd(q, k, v, dout, lse, **kw):
    """Run rpe_attn_bwd once and return (gradients, PreparedBwd) that repeats it in place."""
    g, desc, args, keep = _bwd(q, k, v, dout, lse, **kw)
    return g, PreparedBwd(desc, args, keep, q.device)


def rpe_attn_bwd_noalloc(q, k, v, dout, lse, **kw):
    """rpe_attn_bwd through the allocation-free entry point: the library's own
    device workspace (at most ``_lib.BWD_NOALLOC_MAX_BYTES``) instead of a
    caller workspace; only the gradient tensors are allocated here.  Calls that
    overlap on one GPU race (they share that workspace)."""
    return _bwd(q, k, v, dout, lse, noalloc=True, **kw)[0]


def rpe_attn_bwd(q, k, v, dout, lse, **kw):
    """Gradients of rpe_attn_fwd's output for the output gradient ``dout``.

    ``lse`` is the float32 log-sum-exp the forward returned (return_lse=True).
    Returns a dict of float32 tensors: dq, dk, dv and, for the tables the mode
    and terms use, dbias / drq / drk / drv, shaped as those tables (for every
    map and method: Cross tables of 2S rows and undirected tables of S rows
    are taken and differentiated as they are)."""
    return _bwd(q, k, v, dout, lse, **kw)[0]


def _bwd(q, k, v, dout, lse, *, grid, window=0, prefix_tokens=0, mode="none", terms="", map="swin",
         alpha=0.0, beta=0.0, gamma=0.0, rounding="capped", scale=None, bias=None, rq=None, rk=None,
         rv=None, method="product", noalloc=False):
    torch = _torch()
    if q.dim() != 4 or any(t.shape != q.shape for t in (k, v, dout)):
        raise ValueError("q, k, v, dout must be [B, H, N, d] of one shape")
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q must be bfloat16 or float32")
    if any(t.dtype != q.dtype or not t.is_contiguous() or not t.is_cuda or t.device != q.device
           for t in (q, k, v, dout)):
        raise ValueError("q, k, v, dout must be contiguous device tensors of one dtype and device")
    B, H, N, d = q.shape
    if (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous()
            or lse.device != q.device):
        raise ValueError("lse must be contiguous float32 [B, H, N] on the device of q")
    tabs = [t for t in (bias, rq, rk, rv) if t is not None]
    per_head = any(t.shape[0] == H and H > 1 for t in tabs)
    desc = make_desc(batch=B, heads=H, head_dim=d, grid=grid, window=window, prefix_tokens=prefix_tokens,
                     dtype="bf16" if q.dtype == torch.bfloat16 else "fp32", mode=mode, terms=terms, map=map,
                     alpha=alpha, beta=beta, gamma=gamma, rounding=rounding, scale=scale, tables_per_head=per_head,
                     method=method)
    _check_geometry_and_tables(desc, q, mode, terms, per_head, bias, rq, rk, rv)
    nbytes = ctypes.c_uint64()
    check("rpe_attn_bwd_workspace_size", load().rpe_attn_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(nbytes)))
    ws = None if noalloc else torch.empty(max(1, nbytes.value), dtype=torch.uint8, device=q.device)
    f32 = dict(dtype=torch.float32, device=q.device)
    g = {"dq": torch.empty(q.shape, **f32), "dk": torch.empty(q.shape, **f32), "dv": torch.empty(q.shape, **f32)}
    use = {"bias": mode == "bias", "rq": mode == "contextual" and "q" in terms,
           "rk": mode == "contextual" and "k" in terms, "rv": mode == "contextual" and "v" in terms}
    src = {"bias": bias, "rq": rq, "rk": rk, "rv": rv}
    for n in ("bias", "rq", "rk", "rv"):
        if use[n]:
            if src[n] is None:
                raise ValueError(f"{n} is required by mode {mode!r} and terms {terms!r}")
            g["d" + n] = torch.empty(src[n].shape, **f32)
    gp = lambda n: _ptr(g.get(n))
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse),
            _ptr(bias if use["bias"] else None), _ptr(rq if use["rq"] else None),
            _ptr(rk if use["rk"] else None), _ptr(rv if use["rv"] else None),
            gp("dq"), gp("dk"), gp("dv"), gp("dbias"), gp("drq"), gp("drk"), gp("drv")]
    if noalloc:
        check("rpe_attn_bwd_noalloc", load().rpe_attn_bwd_noalloc(ctypes.byref(desc), *args, _stream(q.device)))
        return g, desc, args, (q, k, v, dout, lse, g, tabs)
    args += [_ptr(ws), ctypes.c_uint64(nbytes.value)]
    check("rpe_attn_bwd", load().rpe_attn_bwd(ctypes.byref(desc), *args, _stream(q.device)))
    return g, desc, args, (q, k, v, dout, lse, ws, g, tabs)
