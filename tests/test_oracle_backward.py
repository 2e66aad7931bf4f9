"""Pins of the oracle's backward (oracle.backward): central finite differences of a separate
forward (reference.recurrence_operator, the transition matrices applied literally), and two
identities of the recurrence ("Recurrent Memory: Write, Erase, Decay, Read", section 05): a
scalar decay commutes with the erase, so both orders give the same gradients, and a scalar gate
is a per-channel gate with equal channels, whose gradient is the sum over the channels."""
import numpy as np
import pytest

from oracle import backward
from oracle import reference as ref

KINDS = [  # (alpha, b, w)
    ("channel", "channel", "channel"), ("scalar", "scalar", "scalar"), ("channel", "scalar", "scalar"),
    ("none", "none", "none"), ("channel", "none", "channel"), ("scalar", "none", "none"),
    ("none", "scalar", "scalar"), ("scalar", "channel", "none"),
]


def draw(kinds, B=1, T=5, H=2, DK=3, DV=2, seed=0, s0=True):
    rng = np.random.default_rng(seed)
    a, b, w = kinds
    gate = lambda kind, width, f: None if kind == "none" else f(
        rng.standard_normal((B, T, H) if kind == "scalar" else (B, T, H, width)))
    sig = lambda z: 1.0 / (1.0 + np.exp(-z))
    x = {
        "q": rng.standard_normal((B, T, H, DK)) * 0.7,
        "k": rng.standard_normal((B, T, H, DK)) * 0.5,
        "v": rng.standard_normal((B, T, H, DV)),
        "log_alpha": gate(a, DK, lambda z: -np.log1p(np.exp(z - 0.5))),
        "b": gate(b, DK, sig),
        "w": gate(w, DV, sig),
        "S0": rng.standard_normal((B, H, DK, DV)) * 0.3 if s0 else None,
    }
    R1 = rng.standard_normal((B, T, H, DV))
    R2 = rng.standard_normal((B, H, DK, DV))
    return x, R1, R2


NAMES = ["q", "k", "v", "log_alpha", "b", "w", "S0"]
GRAD = {"q": "dq", "k": "dk", "v": "dv", "log_alpha": "dlog_alpha", "b": "db", "w": "dw", "S0": "dS0"}


def loss(x, R1, R2, order):
    o, S = ref.recurrence_operator(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], x["S0"],
                                   order=order)
    return float((o * R1).sum() + (S * R2).sum())


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("kinds", KINDS, ids=["-".join(k) for k in KINDS])
def test_backward_matches_finite_differences(kinds, order):
    x, R1, R2 = draw(kinds, seed=3 + order)
    g = backward(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], x["S0"], R1, R2, order=order)
    eps = 1e-6
    for name in NAMES:
        if x[name] is None:
            assert g[GRAD[name]] is None or name == "S0"
            continue
        assert g[GRAD[name]].shape == x[name].shape, name
        flat = x[name].reshape(-1)
        fd = np.empty_like(flat)
        for i in range(flat.size):
            keep = flat[i]
            flat[i] = keep + eps
            lp = loss(x, R1, R2, order)
            flat[i] = keep - eps
            lm = loss(x, R1, R2, order)
            flat[i] = keep
            fd[i] = (lp - lm) / (2 * eps)
        got = g[GRAD[name]].reshape(-1)
        np.testing.assert_allclose(got, fd, rtol=1e-6, atol=1e-7, err_msg=name)


def test_scalar_decay_orders_agree():
    x, R1, R2 = draw(("scalar", "channel", "channel"), T=9, DK=4, DV=3, seed=8)
    g0 = backward(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], x["S0"], R1, R2, order=0)
    g1 = backward(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], x["S0"], R1, R2, order=1)
    for n in GRAD.values():
        np.testing.assert_allclose(g0[n], g1[n], rtol=1e-12, atol=1e-12, err_msg=n)


def test_scalar_gates_are_equal_channels():
    x, R1, R2 = draw(("scalar", "scalar", "scalar"), T=7, DK=4, DV=3, seed=9)
    ex = lambda g, d: np.repeat(g[..., None], d, axis=-1)
    for order in (0, 1):
        gs = backward(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], x["S0"], R1, R2, order=order)
        gc = backward(x["q"], x["k"], x["v"], ex(x["log_alpha"], 4), ex(x["b"], 4), ex(x["w"], 3), x["S0"],
                      R1, R2, order=order)
        for n in ("dq", "dk", "dv", "dS0"):
            np.testing.assert_allclose(gs[n], gc[n], rtol=1e-12, atol=1e-13, err_msg=n)
        for n in ("dlog_alpha", "db", "dw"):
            np.testing.assert_allclose(gs[n], gc[n].sum(-1), rtol=1e-12, atol=1e-13, err_msg=n)
