"""Per-axis index function g(x) of one integer offset x (oracle, fp64).

Test infrastructure only (see the package docstring).

Source: iRPE summary page ("Rethinking and Improving Relative Position
Encoding for Vision Transformer"), Method, eq. 18 and the piecewise index
pseudo-code beside it; Paper vs code, "Non-integer beta"; Pitfalls, "Bucket
edges are sharp" and "Use beta as the code does".

The page states g in words: offsets up to alpha keep their own integer index;
beyond alpha the index grows with log(|x|/alpha)/log(gamma/alpha), scaled so
that it reaches beta at |x| = gamma; the result is capped at beta and rounded
to an integer in [-beta, beta]; the sign of x is kept.

Two readings of the order of "cap" and "round" are provided:

``ROUND_CAPPED`` (default)
    g(x) = sign(x) * rh(min(beta, rh(s(x)))) for |x| > alpha, with rh the
    round-half-away-from-zero of a real number, and a table half-width
    H = rh(beta).  This is the reading under which beta = 3.8 gives 9 index
    values per axis (81 Product buckets) and beta = 7.6 gives 17 (289).

``ROUND_TRUNC``
    g(x) = trunc(sign(x) * min(beta, rh(s(x)))) for |x| > alpha, H = trunc(beta).
    This is the order the page attributes to the released code (the whole
    index truncates toward zero; the table half-width is the integer part of
    beta), giving 7 values per axis at beta = 3.8.

Ties of the rounding are broken away from zero in both readings; the page
does not fix the tie rule.
"""

import math

ROUND_CAPPED = "capped"
ROUND_TRUNC = "trunc"
READINGS = (ROUND_CAPPED, ROUND_TRUNC)


def round_half_away(v):
    """Nearest integer to the real v, halves rounded away from zero."""
    if v >= 0:
        return float(math.floor(v + 0.5))
    return -float(math.floor(-v + 0.5))


def _check_params(alpha, beta, gamma):
    if not (alpha > 0 and gamma > alpha and beta >= alpha):
        raise ValueError(
            f"need alpha > 0, gamma > alpha, beta >= alpha; got {alpha}, {beta}, {gamma}")


def log_position(x, alpha, beta, gamma):
    """The real-valued log-spaced position s(x) used for |x| > alpha (eq. 18)."""
    ax = abs(x)
    return alpha + math.log(ax / alpha) / math.log(gamma / alpha) * (beta - alpha)


def piecewise_index(x, alpha, beta, gamma, reading=ROUND_CAPPED):
    """g(x) for one integer offset x; returns a Python int.

    iRPE summary page, Method, eq. 18 (see module docstring for the readings).
    """
    _check_params(alpha, beta, gamma)
    x = int(x)
    if abs(x) <= alpha:
        return int(round_half_away(float(x)))
    s = log_position(x, alpha, beta, gamma)
    sign = 1.0 if x > 0 else -1.0
    if reading == ROUND_CAPPED:
        return int(sign * round_half_away(min(beta, round_half_away(s))))
    if reading == ROUND_TRUNC:
        return int(math.trunc(sign * min(beta, round_half_away(s))))
    raise ValueError(f"unknown reading {reading!r}")


def half_width(alpha=None, beta=None, gamma=None, reading=ROUND_CAPPED, window=None):
    """Table half-width H: indices lie in [-H, H], S = 2H + 1 per axis.

    Swin window mode (``window`` = M): H = M - 1, since offsets inside an M x M
    window lie in [-(M-1), M-1] (Swin 2D RPE post, section 3.1).
    Piecewise mode: H = rh(beta) (capped reading) or trunc(beta) (truncating
    reading, iRPE page, Pitfalls "Use beta as the code does").
    """
    if window is not None:
        if window < 1:
            raise ValueError("window must be >= 1")
        return window - 1
    _check_params(alpha, beta, gamma)
    if reading == ROUND_CAPPED:
        return int(round_half_away(beta))
    if reading == ROUND_TRUNC:
        return int(math.trunc(beta))
    raise ValueError(f"unknown reading {reading!r}")


def axis_index_table(length, alpha=None, beta=None, gamma=None, reading=ROUND_CAPPED,
                     window=None):
    """g(x) for every offset x in [-(length-1), length-1], in increasing x.

    In Swin window mode the index is the offset itself (Swin 2D RPE post,
    section 3.2: the bias is looked up by the offset, shifted by M-1 only to
    make the array index non-negative, which the bucket id below adds).
    """
    out = []
    for x in range(-(length - 1), length):
        if window is not None:
            out.append(x)
        else:
            out.append(piecewise_index(x, alpha, beta, gamma, reading))
    return out
