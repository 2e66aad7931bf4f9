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


def test_linear_attention_gradients_in_closed_form():
    """With no decay and no erase the read is o_t = q_t (S_0 + sum_{i<=t} k_i^T v_i) ("Recurrent
    Memory: Write, Erase, Decay, Read", section 01: write S <- S + k^T v, read o = q S), so with
    L = <dO, o> + <dS_T, S_T>:
    dq_t = dO_t (S_0 + sum_{i<=t} k_i^T v_i)^T,  dk_i = sum_{t>=i} (dO_t . v_i) q_t + dS_T v_i^T,
    dv_i = sum_{t>=i} (q_t . k_i) dO_t + k_i dS_T,  dS0 = dS_T + sum_t q_t^T dO_t,
    written here with explicit loops, and the write gate w scales v (dw_i = dv_i . v_i)."""
    rng = np.random.default_rng(21)
    B, T, H, DK, DV = 1, 6, 1, 3, 4
    q, k = rng.standard_normal((B, T, H, DK)), rng.standard_normal((B, T, H, DK))
    v, S0 = rng.standard_normal((B, T, H, DV)), rng.standard_normal((B, H, DK, DV))
    dO, dST = rng.standard_normal((B, T, H, DV)), rng.standard_normal((B, H, DK, DV))
    w = np.ones((B, T, H))
    g = backward(q, k, v, None, None, w, S0, dO, dST, order=0)
    Q, K, V, D = q[0, :, 0], k[0, :, 0], v[0, :, 0], dO[0, :, 0]
    s0, dst = S0[0, 0], dST[0, 0]
    dq, dk, dv, ds0 = np.zeros((T, DK)), np.zeros((T, DK)), np.zeros((T, DV)), dst.copy()
    for t in range(T):
        St = s0 + sum(np.outer(K[i], V[i]) for i in range(t + 1))
        dq[t] = St @ D[t]
        ds0 += np.outer(Q[t], D[t])
    for i in range(T):
        dk[i] = sum((D[t] @ V[i]) * Q[t] for t in range(i, T)) + dst @ V[i]
        dv[i] = sum((Q[t] @ K[i]) * D[t] for t in range(i, T)) + K[i] @ dst
    np.testing.assert_allclose(g["dq"][0, :, 0], dq, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dk"][0, :, 0], dk, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dv"][0, :, 0], dv, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dS0"][0, 0], ds0, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dw"][0, :, 0], (dv * V).sum(-1), rtol=1e-12, atol=1e-12)
    assert g["dlog_alpha"] is None and g["db"] is None
