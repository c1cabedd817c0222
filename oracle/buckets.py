"""Attention units, token positions and per-pair bucket ids (oracle).

Test infrastructure only (see the package docstring).

Sources:
* iRPE summary page ("Rethinking and Improving Relative Position Encoding for
  Vision Transformer"), Method: the Product mapping gives one bucket per
  (row index, column index) pair, eq. 25, and the bucket-id pseudo-code
  combines them row first: id = (g(dy) + H) * S + (g(dx) + H).  The class
  token has no grid position (Method, "Other design choices"); here every
  pair that involves a prefix token has no bucket (id -1) and receives no
  position term, which equals the page's extra class-token bucket held at
  its zero initialisation.
* Swin 2D RPE post (深度学习进阶（二十四）Swin 的二维 RPE), sections 3.1-3.2:
  inside an M x M window the 2D offset of two patches is looked up in a
  (2M-1) x (2M-1) table after shifting both components by M-1; the table is
  flattened row by row.  Worked example (M = 3): patch (0,0) attending to
  (2,2) has offset (-2,-2), which lands on cell (0,0).
* Swin relative-bias record (anthology-of-the-sota, SOTA-434), Conditions:
  attention and the bias are restricted to non-overlapping 7 x 7 windows and
  indexed by within-window offsets.

* iRPE page, Method, Cross mapping (eqs. 22-24): a directed mapping with one
  bucket for the row offset and one for the column offset, whose two
  encodings are added; 2 x (2*beta+1) buckets.  The page fixes no order of
  the two halves in one table; here rows [0, S) hold the row-offset
  encodings (index g(dy) + H) and rows [S, 2S) the column-offset encodings
  (index S + g(dx) + H), row part first as in the Product id.

Offset convention: delta = p_query - p_key, rows first (dy, dx); this is the
sign of the Swin post's worked example.
"""

from dataclasses import dataclass, field

from .index import ROUND_CAPPED, half_width, piecewise_index
from .undirected import UNDIRECTED_MAPS, undirected_index

MODES = ("none", "bias", "contextual")
MAPS = ("swin", "piecewise") + UNDIRECTED_MAPS
METHODS = ("product", "cross")


@dataclass(frozen=True)
class Spec:
    """Everything that fixes the computation apart from the tensors.

    grid_h, grid_w : patch grid (tokens in row-major order after any prefix)
    window         : 0 -> one unit is the whole grid; M > 0 -> non-overlapping
                     M x M windows, each its own unit
    prefix         : number of prefix (class) tokens at sequence start (0 or 1)
    mode           : "none" | "bias" | "contextual"
    terms          : subset of {"k", "q", "v"} (contextual mode)
    map            : "swin" (identity index, H = M-1) | "piecewise" (eq. 18), or
                     an undirected map of the offset's distance (see
                     ``oracle.undirected``: "euclidean", "euclidean_rounded",
                     "quantized", "quantized_squared")
    alpha, beta, gamma, reading : piecewise index parameters
    scale          : logit scale s; None -> 1/sqrt(head_dim)
    tables_per_head: True -> one table per head, False -> one shared table
    method         : "product" (one bucket per (row, column) index pair) or
                     "cross" (a row-offset bucket plus a column-offset bucket)
    """

    grid_h: int
    grid_w: int
    window: int = 0
    prefix: int = 0
    mode: str = "none"
    terms: frozenset = field(default_factory=frozenset)
    map: str = "swin"
    alpha: float = 0.0
    beta: float = 0.0
    gamma: float = 0.0
    reading: str = ROUND_CAPPED
    scale: float = None
    tables_per_head: bool = False
    method: str = "product"

    def __post_init__(self):
        if self.mode not in MODES:
            raise ValueError(f"mode {self.mode!r}")
        if self.map not in MAPS:
            raise ValueError(f"map {self.map!r}")
        if self.method not in METHODS:
            raise ValueError(f"method {self.method!r}")
        if self.map in UNDIRECTED_MAPS and self.method != "product":
            raise ValueError("an undirected map has one bucket per pair")
        if self.window:
            if self.grid_h % self.window or self.grid_w % self.window:
                raise ValueError("window must divide the grid")
            if self.prefix:
                raise ValueError("prefix tokens are only defined for global attention")
        if self.mode == "bias" and "v" in self.terms:
            # iRPE page, Method: only the contextual form is defined for values.
            raise ValueError("bias mode has no value term")
        object.__setattr__(self, "terms", frozenset(self.terms))

    # --- sizes -----------------------------------------------------------------
    @property
    def unit_side(self):
        """(rows, cols) of the positioned part of one unit."""
        if self.window:
            return self.window, self.window
        return self.grid_h, self.grid_w

    @property
    def tokens_per_image(self):
        return self.prefix + self.grid_h * self.grid_w

    @property
    def units_per_image(self):
        if self.window:
            return (self.grid_h // self.window) * (self.grid_w // self.window)
        return 1

    @property
    def unit_tokens(self):
        r, c = self.unit_side
        return self.prefix + r * c

    def half_width(self):
        if self.map == "swin":
            r, c = self.unit_side
            return half_width(window=max(r, c))
        return half_width(self.alpha, self.beta, self.gamma, self.reading)

    @property
    def undirected(self):
        return self.map in UNDIRECTED_MAPS

    def g(self, x):
        """Per-axis index of offset x (identity for the Swin map)."""
        if self.undirected:
            raise ValueError("an undirected map has no per-axis index")
        if self.map == "swin":
            return int(x)
        return piecewise_index(x, self.alpha, self.beta, self.gamma, self.reading)

    def u(self, dy, dx):
        """Undirected index in [0, H] of the offset (dy, dx)."""
        return undirected_index(dy, dx, self.map, self.alpha, self.beta, self.gamma, self.reading)


def num_buckets(spec):
    """(H, S, rows): half-width, entries per axis, table rows.

    (2H+1)^2 rows for the Product mapping (iRPE page, Method, "Product");
    (2M-1)^2 for a Swin window (Swin post, section 3.1); 2 (2H+1) for the
    Cross mapping (iRPE page, Method, "Cross"); 2H+1 for the undirected
    maps (eqs. 19-21; only rows H..2H are reached).
    """
    h = spec.half_width()
    s = 2 * h + 1
    if spec.undirected:
        return h, s, s
    return h, s, (2 * s if spec.method == "cross" else s * s)


def unit_positions(spec, unit=0):
    """Token indices (into the N axis) and 2D positions of one unit.

    Returns a list of (token_index, (y, x) or None); prefix tokens come first
    with position None, then the unit's grid tokens in row-major order.
    Positions are grid coordinates; only their differences matter.
    """
    out = []
    for p in range(spec.prefix):
        out.append((p, None))
    if spec.window:
        m = spec.window
        wpr = spec.grid_w // m
        wy, wx = divmod(unit, wpr)
        for r in range(m):
            for c in range(m):
                y, x = wy * m + r, wx * m + c
                out.append((spec.prefix + y * spec.grid_w + x, (y, x)))
    else:
        if unit != 0:
            raise ValueError("global attention has one unit per image")
        for y in range(spec.grid_h):
            for x in range(spec.grid_w):
                out.append((spec.prefix + y * spec.grid_w + x, (y, x)))
    return out


def pair_rows(spec, p_query, p_key):
    """Table rows whose encodings add up to the pair's term: [] if either
    position is None, [Product id] for the Product mapping, [row-offset row,
    column-offset row] for the Cross mapping."""
    if p_query is None or p_key is None:
        return []
    h, s, _ = num_buckets(spec)
    if spec.undirected:
        return [spec.u(p_query[0] - p_key[0], p_query[1] - p_key[1]) + h]
    gy, gx = spec.g(p_query[0] - p_key[0]), spec.g(p_query[1] - p_key[1])
    if not (-h <= gy <= h and -h <= gx <= h):
        raise ValueError(f"index ({gy},{gx}) outside the table half-width {h}")
    if spec.method == "cross":
        return [gy + h, s + gx + h]
    return [(gy + h) * s + (gx + h)]


def pair_bucket(spec, p_query, p_key):
    """Product bucket id of one ordered pair of positions, or -1 if either is None."""
    if p_query is None or p_key is None:
        return -1
    h, s, _ = num_buckets(spec)
    dy = p_query[0] - p_key[0]
    dx = p_query[1] - p_key[1]
    gy, gx = spec.g(dy), spec.g(dx)
    if not (-h <= gy <= h and -h <= gx <= h):
        raise ValueError(f"index ({gy},{gx}) outside the table half-width {h}")
    return (gy + h) * s + (gx + h)


def bucket_map(spec, unit=0):
    """[T][T] list of bucket ids for one unit (query rows, key columns)."""
    toks = unit_positions(spec, unit)
    return [[pair_bucket(spec, pi, pj) for (_, pj) in toks] for (_, pi) in toks]
