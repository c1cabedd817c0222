"""Workload definitions and seeded synthetic inputs.

This module holds shapes, seeds and random draws only: none of the attention
arithmetic.  The same arrays feed the HIP path and the CPU oracle.

The workloads stand in for the pages' benchmarks (ImageNet at 224^2 on a
DeiT-S 14 x 14 patch grid with a class token; Swin-T stage 1 on a 56 x 56
token grid in 7 x 7 windows; a high-resolution 56 x 56 grid), which are not
available here: activations are N(0, 1) and position tables N(0, sigma^2)
with sigma = 0.02 (a discriminating variant uses sigma = 1).

Draw order per workload i (1-based): ``numpy.random.default_rng(1000 + i)``
(``2000 + i`` for the sigma = 1 variant); q, k, v as standard normals of the
full [B, H, N, d] shape, then the present tables in the order bias, rQ, rK,
rV, each sigma * standard normal.  bf16 values are rounded fp64 -> fp32 ->
bf16 (round to nearest even at each step) and handed to both sides as the
same numbers.
"""

from dataclasses import dataclass, field, replace

import numpy as np

BF16 = "bf16"
FP32 = "fp32"


@dataclass(frozen=True)
class Workload:
    index: int                 # 1-based workload number (fixes the seeds)
    name: str
    batch: int
    heads: int
    head_dim: int
    grid_h: int
    grid_w: int
    window: int                # 0: global over the grid
    prefix: int                # class tokens at sequence start
    mode: str                  # "bias" | "contextual"
    terms: frozenset = field(default_factory=frozenset)
    map: str = "swin"          # "swin" | "piecewise"
    alpha: float = 0.0
    beta: float = 0.0
    gamma: float = 0.0
    reading: str = "capped"
    dtype: str = BF16
    table_rows: int = 0        # rows of each position table (S * S)
    tables_per_head: bool = False
    description: str = ""
    method: str = "product"    # "product" | "cross" (table rows: S*S or 2S)

    @property
    def tokens(self):
        return self.prefix + self.grid_h * self.grid_w

    @property
    def qkv_shape(self):
        return (self.batch, self.heads, self.tokens, self.head_dim)

    def resized(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    "swin_tiny": Workload(
        1, "swin_tiny", batch=2, heads=2, head_dim=16, grid_h=4, grid_w=4, window=4,
        prefix=0, mode="bias", map="swin", dtype=FP32, table_rows=49, tables_per_head=True,
        description="Swin window bias, one 4x4 window, B2 h2 d16 fp32, 7x7 table per head"),
    "swin_t_w7": Workload(
        2, "swin_t_w7", batch=32, heads=3, head_dim=32, grid_h=56, grid_w=56, window=7,
        prefix=0, mode="bias", map="swin", dtype=BF16, table_rows=169, tables_per_head=True,
        description="Swin-T stage-1 window attention: B32, 56x56 grid, 7x7 windows, h3 d32 bf16, "
                    "13x13 bias table per head"),
    "deit_s_irpe_k": Workload(
        3, "deit_s_irpe_k", batch=64, heads=6, head_dim=64, grid_h=14, grid_w=14, window=0,
        prefix=1, mode="contextual", terms=frozenset("k"), map="piecewise",
        alpha=1.9, beta=3.8, gamma=15.2, dtype=BF16, table_rows=81, tables_per_head=False,
        description="DeiT-S iRPE contextual product on keys: B64, 14x14+cls (197 tokens), "
                    "h6 d64 bf16, r^K 81x64 shared"),
    "deit_s_irpe_qkv": Workload(
        4, "deit_s_irpe_qkv", batch=64, heads=6, head_dim=64, grid_h=14, grid_w=14, window=0,
        prefix=1, mode="contextual", terms=frozenset("qkv"), map="piecewise",
        alpha=1.9, beta=3.8, gamma=15.2, dtype=BF16, table_rows=81, tables_per_head=False,
        description="DeiT-S iRPE contextual product on queries, keys and values: "
                    "B64, 197 tokens, h6 d64 bf16, r^Q r^K r^V 81x64 shared"),
    "highres_irpe_k": Workload(
        5, "highres_irpe_k", batch=4, heads=6, head_dim=64, grid_h=56, grid_w=56, window=0,
        prefix=0, mode="contextual", terms=frozenset("k"), map="piecewise",
        alpha=3.8, beta=7.6, gamma=30.4, dtype=BF16, table_rows=289, tables_per_head=False,
        description="High-resolution iRPE on keys: B4, 56x56 grid (3136 tokens), h6 d64 bf16, "
                    "r^K 289x64 shared"),
    # The mode and mapping variants the kernel also runs (measured as secondaries).
    "deit_s_irpe_bias": Workload(
        6, "deit_s_irpe_bias", batch=64, heads=6, head_dim=64, grid_h=14, grid_w=14, window=0,
        prefix=1, mode="bias", map="piecewise", alpha=1.9, beta=3.8, gamma=15.2, dtype=BF16,
        table_rows=81, tables_per_head=True,
        description="DeiT-S iRPE bias mode: B64, 14x14+cls (197 tokens), h6 d64 bf16, 81-entry bias per head"),
    "deit_s_irpe_k_cross": Workload(
        7, "deit_s_irpe_k_cross", batch=64, heads=6, head_dim=64, grid_h=14, grid_w=14, window=0,
        prefix=1, mode="contextual", terms=frozenset("k"), map="piecewise", alpha=1.9, beta=3.8,
        gamma=15.2, dtype=BF16, table_rows=18, tables_per_head=False, method="cross",
        description="DeiT-S iRPE contextual Cross mapping on keys: B64, 197 tokens, h6 d64 bf16, "
                    "r^K 18x64 (9 row + 9 column) shared"),
    "detr_irpe_k": Workload(
        8, "detr_irpe_k", batch=8, heads=8, head_dim=32, grid_h=25, grid_w=38, window=0,
        prefix=0, mode="contextual", terms=frozenset("k"), map="piecewise", alpha=1.9, beta=3.8,
        gamma=15.2, dtype=BF16, table_rows=81, tables_per_head=False,
        description="DETR-like encoder iRPE on keys, non-square 25x38 grid (950 tokens, an 800x1216 "
                    "image at stride 32): B8, h8 d32 bf16, r^K 81x32 shared"),
    "detr_wide_irpe_k": Workload(
        10, "detr_wide_irpe_k", batch=2, heads=8, head_dim=32, grid_h=50, grid_w=84, window=0,
        prefix=0, mode="contextual", terms=frozenset("k"), map="piecewise", alpha=1.9, beta=3.8,
        gamma=15.2, dtype=BF16, table_rows=81, tables_per_head=False,
        description="DETR-like encoder iRPE on keys at stride 16: 50x84 grid (4200 tokens, an 800x1344 "
                    "image; rows of 84 columns), B2, h8 d32 bf16, r^K 81x32 shared"),
    "swin_t_w7_irpe_qkv": Workload(
        11, "swin_t_w7_irpe_qkv", batch=32, heads=3, head_dim=32, grid_h=56, grid_w=56, window=7,
        prefix=0, mode="contextual", terms=frozenset("kqv"), map="piecewise", alpha=1.9, beta=3.8,
        gamma=15.2, dtype=BF16, table_rows=81, tables_per_head=False,
        description="Swin-T stage-1 7x7 windows with iRPE contextual product on queries, keys and values: "
                    "B32, 56x56 grid (64 windows of 49 tokens), h3 d32 bf16, r^Q, r^K, r^V 81x32 shared"),
    "deit_s_irpe_bias_euclid": Workload(
        9, "deit_s_irpe_bias_euclid", batch=64, heads=6, head_dim=64, grid_h=14, grid_w=14, window=0,
        prefix=1, mode="bias", map="euclidean", alpha=1.9, beta=3.8, gamma=15.2, dtype=BF16,
        table_rows=9, tables_per_head=True,
        description="DeiT-S iRPE bias mode with the undirected Euclidean mapping: B64, 197 tokens, "
                    "h6 d64 bf16, 9-entry bias per head"),
}


def round_to_dtype(x, dtype):
    """Round float64 values to the storage dtype, returned as float64."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == FP32:
        return x.astype(np.float32).astype(np.float64)
    if dtype == BF16:
        import torch
        t = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
        return t.to(torch.float64).numpy()
    raise ValueError(dtype)


def make_inputs(w, sigma=0.02, seed=None, rng=None):
    """Seeded inputs for workload ``w`` as float64 arrays of dtype-exact values.

    Returns a dict with q, k, v ([B, H, N, d]) and the tables the workload
    uses: bias ([H or 1][rows], always fp32 values), rq / rk / rv
    ([H or 1][rows][d], values of the workload dtype).
    """
    if rng is None:
        if seed is None:
            seed = 1000 + w.index if sigma == 0.02 else 2000 + w.index
        rng = np.random.default_rng(seed)
    shape = w.qkv_shape
    out = {}
    for name in ("q", "k", "v"):
        out[name] = round_to_dtype(rng.standard_normal(shape), w.dtype)
    th = w.heads if w.tables_per_head else 1
    if w.mode == "bias":
        out["bias"] = round_to_dtype(sigma * rng.standard_normal((th, w.table_rows)), FP32)
    if w.mode == "contextual":
        for term in ("q", "k", "v"):
            if term in w.terms:
                out["r" + term] = round_to_dtype(
                    sigma * rng.standard_normal((th, w.table_rows, w.head_dim)), w.dtype)
    return out
