"""Pins of the oracle's backward pass (CPU only): central finite differences of
the forward oracle, which is pinned on its own, and torch's autograd of a
library softmax attention for the case without position terms."""

import numpy as np
import pytest
import torch

from oracle import Spec, attention, num_buckets
from oracle.backward import attention_backward

CASES = [
    Spec(3, 4, prefix=1, mode="contextual", terms={"k", "q", "v"}, map="piecewise", alpha=0.9, beta=1.7,
         gamma=3.0, tables_per_head=True),
    Spec(2, 3, mode="contextual", terms={"k"}, map="piecewise", alpha=1.0, beta=2.0, gamma=8.0),
    Spec(4, 4, window=2, mode="bias", map="swin", tables_per_head=True),
    Spec(3, 3, prefix=2, mode="bias", map="piecewise", alpha=1.0, beta=2.0, gamma=4.0),
    Spec(2, 4, prefix=1, mode="contextual", terms={"q", "v"}, map="piecewise", alpha=1.0, beta=2.0, gamma=4.0,
         method="cross"),
    Spec(3, 3, mode="none", scale=0.7),
    Spec(3, 3, prefix=1, mode="contextual", terms={"k"}, map="piecewise", alpha=1.0, beta=2.0, gamma=4.0,
         method="cross", tables_per_head=True),
    Spec(3, 4, mode="bias", map="piecewise", alpha=1.0, beta=2.0, gamma=4.0, method="cross"),
    Spec(3, 3, prefix=1, mode="bias", map="euclidean", alpha=1.0, beta=2.0, gamma=4.0, tables_per_head=True),
    Spec(3, 4, mode="contextual", terms={"k", "v"}, map="quantized", alpha=1.0, beta=2.0, gamma=4.0),
]


def _setup(spec, rng, B=1, H=2, d=4):
    N = spec.tokens_per_image
    x = {n: rng.standard_normal((B, H, N, d)) for n in ("q", "k", "v", "do")}
    _, _, nb = num_buckets(spec)
    th = H if spec.tables_per_head else 1
    tabs = {}
    if spec.mode == "bias":
        tabs["bias"] = rng.standard_normal((th, nb))
    if spec.mode == "contextual":
        for t in sorted(spec.terms):
            tabs["r" + t] = rng.standard_normal((th, nb, d))
    return x, tabs


@pytest.mark.parametrize("spec", CASES)
def test_backward_matches_finite_differences(spec):
    rng = np.random.default_rng(3)
    x, tabs = _setup(spec, rng)
    g = attention_backward(spec, x["q"], x["k"], x["v"], x["do"], **tabs)

    def loss(over):
        args = {n: over.get(n, x[n]) for n in ("q", "k", "v")}
        t = {n: over.get(n, a) for n, a in tabs.items()}
        o, _ = attention(spec, args["q"], args["k"], args["v"], **t)
        return float((o * x["do"]).sum())

    eps = 1e-6
    names = [("q", "dq"), ("k", "dk"), ("v", "dv")] + [(n, "d" + n) for n in tabs]
    for name, key in names:
        arr = x[name] if name in x else tabs[name]
        num = np.zeros_like(arr)
        for ix in np.ndindex(arr.shape):
            a1, a2 = arr.copy(), arr.copy()
            a1[ix] += eps
            a2[ix] -= eps
            num[ix] = (loss({name: a1}) - loss({name: a2})) / (2 * eps)
        err = np.abs(num - g[key]).max()
        assert err <= 1e-6 * max(1.0, np.abs(num).max()), (name, err)


def test_backward_without_position_terms_matches_autograd():
    spec = Spec(3, 5, prefix=1, mode="none")
    rng = np.random.default_rng(5)
    x, _ = _setup(spec, rng, B=2, H=3, d=6)
    g = attention_backward(spec, x["q"], x["k"], x["v"], x["do"])
    t = {n: torch.tensor(x[n], requires_grad=True) for n in ("q", "k", "v")}
    o = torch.nn.functional.scaled_dot_product_attention(t["q"], t["k"], t["v"], scale=1 / np.sqrt(6))
    (o * torch.tensor(x["do"])).sum().backward()
    for n in ("q", "k", "v"):
        np.testing.assert_allclose(g["d" + n], t[n].grad.numpy(), atol=1e-12)
