"""Pins for the CPU oracle: each test checks the C fp64 recurrence against something the
pages or the mathematics fix, not against a retyping of its own loop.

Page titles cited: [RM] "Recurrent Memory: Write, Erase, Decay, Read";
[ET] "The Eraser Trilogy"; [HLAR] "How Linear Attention Remembers" (summary page);
[GDN2] the Gated DeltaNet-2 abstract.
"""
import numpy as np
import pytest

import oracle
from oracle import reference as ref

RNG = np.random.default_rng(20260101)


def unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rand_case(B=2, T=37, H=2, DK=6, DV=5, alpha="channel", b="channel", w="channel", seed=0,
              s0=True, mu=-1.0):
    r = np.random.default_rng(seed)
    q = unit_rows(r.standard_normal((B, T, H, DK)))
    k = unit_rows(r.standard_normal((B, T, H, DK)))
    v = r.standard_normal((B, T, H, DV))
    shp = {"none": None, "scalar": (B, T, H), "channel_k": (B, T, H, DK), "channel_v": (B, T, H, DV)}
    la = None if alpha == "none" else -np.log1p(np.exp(-(r.standard_normal(
        shp["scalar" if alpha == "scalar" else "channel_k"]) + mu)))
    bb = None if b == "none" else 1 / (1 + np.exp(-r.standard_normal(
        shp["scalar" if b == "scalar" else "channel_k"])))
    ww = None if w == "none" else 1 / (1 + np.exp(-r.standard_normal(
        shp["scalar" if w == "scalar" else "channel_v"])))
    S0 = 0.3 * r.standard_normal((B, H, DK, DV)) if s0 else None
    f = lambda a: None if a is None else a.astype(np.float32)
    return dict(q=f(q), k=f(k), v=f(v), log_alpha=f(la), b=f(bb), w=f(ww), S0=S0)


def run(case, order=0):
    return oracle.forward(case["q"], case["k"], case["v"], case["log_alpha"], case["b"], case["w"],
                          case["S0"], order=order)


# ---------------------------------------------------------------- write and read


def test_single_write_readback_is_norm_squared_times_v():
    """[RM] section 01: after S <- S + k^T v, reading with the same key gives ||k||^2 v.
    d_k != d_v so that a transposed write or read cannot pass."""
    k = RNG.standard_normal((1, 1, 1, 5)).astype(np.float32)
    v = RNG.standard_normal((1, 1, 1, 3)).astype(np.float32)
    o, S = oracle.forward(k, k, v)
    kk = float((k.astype(np.float64) ** 2).sum())
    np.testing.assert_allclose(o[0, 0, 0], kk * v[0, 0, 0].astype(np.float64), rtol=1e-14)
    np.testing.assert_allclose(S[0, 0], np.outer(k[0, 0, 0].astype(np.float64), v[0, 0, 0]), rtol=1e-14)


def test_read_sees_this_tokens_write():
    """[HLAR] Analytical Framework: o_t = q_t^T S_t, the state after token t's update.
    With S0 = 0 and one token, o_1 = (q . k) v exactly."""
    q = RNG.standard_normal((1, 1, 1, 4)).astype(np.float32)
    k = RNG.standard_normal((1, 1, 1, 4)).astype(np.float32)
    v = RNG.standard_normal((1, 1, 1, 7)).astype(np.float32)
    o, _ = oracle.forward(q, k, v)
    qk = float(q.astype(np.float64).ravel() @ k.astype(np.float64).ravel())
    np.testing.assert_allclose(o[0, 0, 0], qk * v[0, 0, 0].astype(np.float64), rtol=1e-14)


# ---------------------------------------------------------------- the erase


def test_overwrite_returns_latest_value():
    """[RM] section 02 problem one and [ET] Eraser two: writing the same unit key twice
    with beta = 1 leaves the second value, whatever was stored before."""
    DK, DV = 6, 4
    k1 = unit_rows(RNG.standard_normal(DK))
    k = np.stack([k1, k1]).reshape(1, 2, 1, DK).astype(np.float32)
    v = RNG.standard_normal((1, 2, 1, DV)).astype(np.float32)
    beta = np.ones((1, 2, 1), np.float32)
    S0 = RNG.standard_normal((1, 1, DK, DV))
    o, S = oracle.forward(k, k, v, None, beta, beta, S0)
    kd = k[0, 0, 0].astype(np.float64)
    np.testing.assert_allclose(kd @ S[0, 0], v[0, 1, 0], atol=1e-6)  # |k| = 1 in float32
    np.testing.assert_allclose(o[0, 1, 0], v[0, 1, 0], atol=1e-6)
    # pure accumulation instead returns the sum (plus the old content): the problem the
    # erase exists to fix
    o_add, _ = oracle.forward(k, k, v)
    np.testing.assert_allclose(o_add[0, 1, 0], v[0, 0, 0] + v[0, 1, 0], atol=1e-6)


@pytest.mark.parametrize("rule", ["add", "delta"])
def test_orthogonal_keys_recall_exactly(rule):
    """[RM] section 02 problem two: at most d mutually orthogonal keys fit in a d x d board,
    and each reads back its own value exactly; with beta = 1 the delta rule does too."""
    d, DV = 8, 5
    Qm, _ = np.linalg.qr(RNG.standard_normal((d, d)))
    keys = Qm.T  # rows orthonormal (in fp64)
    # fp32 inputs: orthonormal up to ~1e-7, so recall is exact up to that
    k = keys.reshape(1, d, 1, d).astype(np.float32)
    v = RNG.standard_normal((1, d, 1, DV)).astype(np.float32)
    beta = np.ones((1, d, 1), np.float32) if rule == "delta" else None
    _, S = oracle.forward(k, k, v, None, beta, beta)
    recall = k[0, :, 0].astype(np.float64) @ S[0, 0]
    np.testing.assert_allclose(recall, v[0, :, 0], atol=2e-6)


def test_more_keys_than_dimensions_cross_talk():
    """[RM] section 02: the (d+1)-th key has nonzero overlap with something stored, so pure
    accumulation cannot recall every value."""
    d, DV = 6, 4
    k = unit_rows(RNG.standard_normal((d + 1, d))).reshape(1, d + 1, 1, d).astype(np.float32)
    v = RNG.standard_normal((1, d + 1, 1, DV)).astype(np.float32)
    _, S = oracle.forward(k, k, v)
    recall = k[0, :, 0].astype(np.float64) @ S[0, 0]
    assert np.abs(recall - v[0, :, 0]).max() > 0.05


def _erase_only(k, beta, S0):
    """One token with the write off (w = 0) and no decay."""
    DK = k.shape[-1]
    DV = S0.shape[-1]
    kk = k.reshape(1, -1, 1, DK).astype(np.float32)
    T = kk.shape[1]
    bb = np.full((1, T, 1), beta, np.float32)
    zero = np.zeros((1, T, 1), np.float32)
    v = np.zeros((1, T, 1, DV), np.float32)
    return oracle.forward(kk, kk, v, None, bb, zero, S0.reshape(1, 1, DK, DV))[1][0, 0]


def test_erase_beta1_is_orthogonal_projection():
    """[RM] section 03: at beta = 1 the erase (I - k^T k) annihilates the k direction, leaves
    every direction orthogonal to k untouched, and is idempotent."""
    DK, DV = 5, 3
    k = np.array([1.0, 1.0, 0.0, 0.0, 0.0]) / 2 ** 0.5
    k32 = k.astype(np.float32).astype(np.float64)
    S0 = RNG.standard_normal((DK, DV))
    S1 = _erase_only(k, 1.0, S0)
    np.testing.assert_allclose(k32 @ S1, 0.0, atol=1e-7)
    z = np.array([1.0, -1.0, 0.3, -2.0, 0.5])  # z . k = 0 exactly
    np.testing.assert_allclose(z @ S1, z @ S0, rtol=1e-12, atol=1e-12)
    S2 = _erase_only(np.stack([k, k]), 1.0, S0)
    np.testing.assert_allclose(S2, S1, atol=1e-7)


def test_erase_beta2_is_reflection():
    """[RM] section 03: at beta = 2 the operator is a Householder reflection: it keeps the
    Frobenius norm and applying it twice gives back the state."""
    DK, DV = 4, 6
    k = np.array([0.5, 0.5, 0.5, 0.5])  # unit, exact in binary
    S0 = RNG.standard_normal((DK, DV))
    S1 = _erase_only(k, 2.0, S0)
    np.testing.assert_allclose(np.linalg.norm(S1), np.linalg.norm(S0), rtol=1e-14)
    S2 = _erase_only(np.stack([k, k]), 2.0, S0)
    np.testing.assert_allclose(S2, S0, atol=1e-13)
    assert np.abs(S1 - S0).max() > 0.1


def test_erase_gate_is_on_the_key_side():
    """[GDN2]: the channel-wise erase gate b_t acts on the key side.  With the write off,
    S1 = (I - k^T (b . k)) S0, so a query z with z . k = 0 is untouched and the read along
    c = b . k is scaled by (1 - c . k).  Putting b on the wrong factor fails both."""
    DK, DV = 4, 3
    k = np.array([1.0, 1.0, 0.0, 0.0]).reshape(1, 1, 1, DK).astype(np.float32)
    b = np.array([1.0, 0.25, 0.5, 0.75]).reshape(1, 1, 1, DK).astype(np.float32)
    w = np.zeros((1, 1, 1, DV), np.float32)
    v = np.ones((1, 1, 1, DV), np.float32)
    S0 = RNG.standard_normal((1, 1, DK, DV))
    _, S = oracle.forward(k, k, v, None, b, w, S0)
    c = (b * k)[0, 0, 0].astype(np.float64)
    kd = k[0, 0, 0].astype(np.float64)
    z = np.array([1.0, -1.0, 2.0, 3.0])  # z . k = 0
    np.testing.assert_allclose(z @ S[0, 0], z @ S0[0, 0], rtol=1e-13)
    np.testing.assert_allclose(c @ S[0, 0], (1 - c @ kd) * (c @ S0[0, 0]), rtol=1e-13)


def test_delta_step_is_one_sgd_step():
    """[ET] Eraser two: one delta-rule step is one step of gradient descent on
    1/2 ||k S - v||^2 with learning rate beta.  The gradient comes from autograd."""
    import torch
    DK, DV = 6, 4
    k = unit_rows(RNG.standard_normal(DK)).astype(np.float32)
    v = RNG.standard_normal(DV).astype(np.float32)
    beta = np.float32(0.37)
    S0 = RNG.standard_normal((DK, DV))
    St = torch.tensor(S0, dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k, dtype=torch.float64)
    vt = torch.tensor(v, dtype=torch.float64)
    loss = 0.5 * ((kt @ St - vt) ** 2).sum()
    loss.backward()
    expect = S0 - float(beta) * St.grad.numpy()
    bb = np.full((1, 1, 1), beta, np.float32)
    _, S = oracle.forward(k.reshape(1, 1, 1, DK), k.reshape(1, 1, 1, DK), v.reshape(1, 1, 1, DV),
                          None, bb, bb, S0.reshape(1, 1, DK, DV))
    np.testing.assert_allclose(S[0, 0], expect, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- the decay


@pytest.mark.parametrize("kind", ["scalar", "channel"])
def test_decay_survival_is_exp_of_log_sum(kind):
    """[RM] section 04: a write at token x survives to token x+t with factor
    prod alpha = exp(sum log alpha), taken over the decays applied after the write
    (tokens x+1 .. x+t under the unified equation; the write is not decayed at x)."""
    T, DK, DV, x = 9, 4, 3, 3
    k = unit_rows(RNG.standard_normal((1, T, 1, DK))).astype(np.float32)
    v = RNG.standard_normal((1, T, 1, DV)).astype(np.float32)
    w = np.zeros((1, T, 1), np.float32)
    w[0, x, 0] = 1.0  # only token x writes
    shp = (1, T, 1) if kind == "scalar" else (1, T, 1, DK)
    la = (-np.abs(RNG.standard_normal(shp)) * 0.7).astype(np.float32)
    _, S = oracle.forward(k, k, v, la, None, w)
    surv = np.exp(la[0, x + 1:, 0].astype(np.float64).sum(axis=0))
    surv = np.broadcast_to(surv, (DK,)) if kind == "scalar" else surv
    expect = surv[:, None] * np.outer(k[0, x, 0].astype(np.float64), v[0, x, 0])
    np.testing.assert_allclose(S[0, 0], expect, rtol=1e-12)


def test_worked_example_erase_then_decay_order():
    """[RM] section 05 writes Diag(alpha)(I - beta k^T k) S + beta k^T v: erase, then decay,
    then an undecayed write.  Hand-derived 2x2 case (exact in binary):
    k = (1, 1), beta = 1/2 (so I - beta k^T k = [[.5, -.5], [-.5, .5]]), alpha = (1, 1/2),
    S0 = I, v = (1, 2), write beta k^T v = [[.5, 1], [.5, 1]]:
      erase then decay:  [[.5, -.5], [-.25, .25]] + [[.5, 1], [.5, 1]] = [[1, .5], [.25, 1.25]]
      decay then erase:  [[.5, -.25], [-.5, .25]] + [[.5, 1], [.5, 1]] = [[1, .75], [0, 1.25]]"""
    k = np.array([1.0, 1.0], np.float32).reshape(1, 1, 1, 2)
    v = np.array([1.0, 2.0], np.float32).reshape(1, 1, 1, 2)
    la = np.log(np.array([1.0, 0.5])).astype(np.float32).reshape(1, 1, 1, 2)
    half = np.full((1, 1, 1), 0.5, np.float32)
    S0 = np.eye(2).reshape(1, 1, 2, 2)
    _, S_ed = oracle.forward(k, k, v, la, half, half, S0, order=oracle.ORDER_ERASE_THEN_DECAY)
    _, S_de = oracle.forward(k, k, v, la, half, half, S0, order=oracle.ORDER_DECAY_THEN_ERASE)
    np.testing.assert_allclose(S_ed[0, 0], [[1.0, 0.5], [0.25, 1.25]], atol=1e-7)
    np.testing.assert_allclose(S_de[0, 0], [[1.0, 0.75], [0.0, 1.25]], atol=1e-7)


def test_orders_agree_for_scalar_decay_and_differ_for_channel_decay():
    """A scalar alpha commutes with the erase, a per-channel one does not."""
    c = rand_case(alpha="scalar", seed=3)
    o0, S0_ = run(c, 0)
    o1, S1_ = run(c, 1)
    np.testing.assert_allclose(o0, o1, rtol=1e-11, atol=1e-12)
    c = rand_case(alpha="channel", seed=3)
    o0, _ = run(c, 0)
    o1, _ = run(c, 1)
    assert np.abs(o0 - o1).max() > 1e-3


# ---------------------------------------------------------------- the family


def test_reduces_to_linear_attention():
    """[RM] section 05: erase off and alpha = 1 is 2020 linear attention; [ET] The Rosetta
    Stone: its masked-matrix form is O = tril(Q K^T) V."""
    c = rand_case(alpha="none", b="none", w="none", s0=False, seed=4)
    o, _ = run(c)
    np.testing.assert_allclose(o, ref.linear_attention_masked(c["q"], c["k"], c["v"]), rtol=1e-11,
                               atol=1e-12)


@pytest.mark.parametrize("kind", ["scalar", "channel"])
def test_reduces_to_gated_linear_attention(kind):
    """[RM] section 05 / [ET] Eraser one: erase off with a decay is GLA (per-channel) or the
    Mamba-2 shape (scalar).  Masked form with the exact pairwise decay exp(G_t - G_i); the
    write gate w scales v on the value side."""
    c = rand_case(alpha=kind, b="none", w="channel", s0=False, seed=5)
    o, _ = run(c)
    x = c["w"].astype(np.float64) * c["v"]
    np.testing.assert_allclose(o, ref.gla_masked(c["q"], c["k"], x, c["log_alpha"]), rtol=1e-10,
                               atol=1e-12)


def test_reduces_to_deltanet_three_lines():
    """[RM] section 03: alpha = 1, b = w = beta is the three-line delta rule."""
    c = rand_case(alpha="none", b="scalar", w="scalar", seed=6)
    c["w"] = c["b"]
    o, S = run(c)
    o3, S3 = ref.deltanet_three_line(c["q"], c["k"], c["v"], c["b"], c["S0"])
    np.testing.assert_allclose(o, o3, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S, S3, rtol=1e-11, atol=1e-12)


def test_gdn2_reduces_to_kda_and_kda_to_gdn():
    """[GDN2]: Gated DeltaNet-2 reduces to KDA when b and w collapse to one scalar beta, and to
    Gated DeltaNet when the decay collapses to a scalar as well."""
    c = rand_case(alpha="channel", b="scalar", w="scalar", seed=7)
    c["w"] = c["b"]
    o_kda, S_kda = run(c)
    g = dict(c)
    g["b"] = np.repeat(c["b"][..., None], c["q"].shape[-1], axis=-1)
    g["w"] = np.repeat(c["b"][..., None], c["v"].shape[-1], axis=-1)
    o_g2, S_g2 = run(g)
    np.testing.assert_allclose(o_g2, o_kda, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(S_g2, S_kda, rtol=1e-13, atol=1e-14)
    s = dict(c)
    s["log_alpha"] = c["log_alpha"][..., 0].copy()
    o_gdn, _ = run(s)
    k = dict(c)
    k["log_alpha"] = np.repeat(s["log_alpha"][..., None], c["q"].shape[-1], axis=-1)
    o_kda2, _ = run(k)
    np.testing.assert_allclose(o_kda2, o_gdn, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("kinds", [("channel", "channel", "channel"), ("scalar", "scalar", "scalar"),
                                   ("channel", "scalar", "channel"), ("none", "channel", "none"),
                                   ("scalar", "none", "scalar")])
def test_matches_operator_form_twin(order, kinds):
    """The C loop equals the NumPy twin that applies the unified equation as an explicit
    dk x dk transition matrix (independent code, same definition)."""
    a, b, w = kinds
    c = rand_case(alpha=a, b=b, w=w, seed=11 + order)
    o, S = run(c, order)
    o2, S2 = ref.recurrence_operator(c["q"], c["k"], c["v"], c["log_alpha"], c["b"], c["w"], c["S0"],
                                     order)
    np.testing.assert_allclose(o, o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S, S2, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- structure


def test_linearity_and_decomposition():
    """[HLAR] Analytical Framework: S_t = T_t(S_{t-1}) + W_t with T_t linear, so the state is
    a sum of per-position contributions; with fixed keys and gates the map
    (S0, v) -> (o, S_T) is linear: f(S0, v1 + v2) = f(S0, v1) + f(0, v2)."""
    c1 = rand_case(seed=21)
    c2 = dict(c1)
    c2["v"] = np.random.default_rng(22).standard_normal(c1["v"].shape).astype(np.float32)
    both = dict(c1)
    both["v"] = (c1["v"].astype(np.float64) + c2["v"]).astype(np.float32)
    # keep v1 + v2 exact: use values on a coarse grid
    for d in (c1, c2):
        d["v"] = np.round(d["v"] * 64) / 64
    both["v"] = c1["v"] + c2["v"]
    c2["S0"] = None
    o_b, S_b = run(both)
    o_1, S_1 = run(c1)
    o_2, S_2 = run(c2)
    np.testing.assert_allclose(o_b, o_1 + o_2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S_b, S_1 + S_2, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("order", [0, 1])
def test_contributions_sum_to_the_state(order):
    """[HLAR] Analytical Framework: S_t = sum_{i <= t} C_i^(t) from a zero state, where
    C_i^(t) = (T_t o ... o T_{i+1})(W_i).  The reference contributions (transition operators
    composed from the definition) must add up to the C oracle's state at every t tested, and
    a write blocked at x (w_x = 0) must leave S_t - C_x^(t)."""
    c = rand_case(B=1, T=23, H=2, seed=31, s0=False)
    for t in (0, 9, 22):
        cut = {n: (None if a is None else a[:, :t + 1]) for n, a in c.items() if n != "S0"}
        _, S = oracle.forward(cut["q"], cut["k"], cut["v"], cut["log_alpha"], cut["b"], cut["w"],
                              None, order=order)
        total = sum(ref.contribution(c["q"], c["k"], c["v"], c["log_alpha"], c["b"], c["w"],
                                     i=i, t=t, order=order) for i in range(t + 1))
        np.testing.assert_allclose(total, S, rtol=1e-10, atol=1e-12)
    x, t = 5, 22
    wb = c["w"].copy()
    wb[:, x] = 0
    _, S = oracle.forward(c["q"], c["k"], c["v"], c["log_alpha"], c["b"], c["w"], None, order=order)
    _, Sb = oracle.forward(c["q"], c["k"], c["v"], c["log_alpha"], c["b"], wb, None, order=order)
    Cx = ref.contribution(c["q"], c["k"], c["v"], c["log_alpha"], c["b"], c["w"], i=x, t=t, order=order)
    np.testing.assert_allclose(Sb, S - Cx, rtol=1e-10, atol=1e-12)
    # the contribution of the last token is its own write, k_t^T (w_t . v_t)
    Ct = ref.contribution(c["q"], c["k"], c["v"], c["log_alpha"], c["b"], c["w"], i=t, t=t, order=order)
    W = np.einsum("bhk,bhv->bhkv", c["k"][:, t].astype(np.float64),
                  c["w"][:, t].astype(np.float64) * c["v"][:, t].astype(np.float64))
    np.testing.assert_allclose(Ct, W, rtol=1e-12, atol=1e-14)


def test_resume_from_intermediate_state():
    """[HLAR]: S_t depends only on S_{t-1} and token t, so running [0, T1) and then [T1, T)
    from the state reached equals one run."""
    c = rand_case(T=41, seed=23)
    o, S = run(c)
    T1 = 17
    first = {n: (a[:, :T1] if (a is not None and n != "S0") else a) for n, a in c.items()}
    second = {n: (a[:, T1:] if (a is not None and n != "S0") else a) for n, a in c.items()}
    oa, Sa = run(first)
    second["S0"] = Sa
    ob, Sb = run(second)
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=1), o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Sb, S, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("chunk", [4, 16, 64])
@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("kinds", [("channel", "channel", "channel"), ("scalar", "scalar", "scalar"),
                                   ("channel", "scalar", "scalar"), ("none", "channel", "channel")])
def test_chunkwise_equals_recurrence(chunk, order, kinds):
    """[RM] section 03: the erase is linear, so it reassociates into a chunkwise-parallel
    form; [RM] section 04: gating enters it as prefix sums of log alpha.  The chunk (WY) form
    in fp64 equals the token-by-token recurrence on tiny inputs, T not a multiple of the
    chunk."""
    a, b, w = kinds
    c = rand_case(T=70, DK=8, DV=6, alpha=a, b=b, w=w, seed=31 + chunk + order)
    o, S = run(c, order)
    oc, Sc = ref.chunkwise(c["q"], c["k"], c["v"], c["log_alpha"], c["b"], c["w"], c["S0"], order,
                           chunk)
    np.testing.assert_allclose(oc, o, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(Sc, S, rtol=1e-10, atol=1e-11)


def test_columns_are_independent():
    """[RM] section 05: the transition multiplies S from the left, so each value column
    evolves on its own: permuting v and w columns permutes o and S columns."""
    c = rand_case(DV=7, seed=41)
    perm = np.array([3, 0, 6, 1, 5, 2, 4])
    p = dict(c)
    p["v"] = c["v"][..., perm].copy()
    p["w"] = c["w"][..., perm].copy()
    p["S0"] = c["S0"][..., perm].copy()
    o, S = run(c)
    op, Sp = run(p)
    np.testing.assert_array_equal(op, o[..., perm])
    np.testing.assert_array_equal(Sp, S[..., perm])


def test_thread_count_does_not_change_results():
    c = rand_case(B=1, H=1, T=33, DK=8, DV=32, seed=43)
    a = oracle.forward(c["q"], c["k"], c["v"], c["log_alpha"], c["b"], c["w"], c["S0"], n_threads=1)
    b = oracle.forward(c["q"], c["k"], c["v"], c["log_alpha"], c["b"], c["w"], c["S0"], n_threads=8)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_oracle_rejects_bad_arguments():
    q = np.zeros((1, 1, 1, 4), np.float32)
    with pytest.raises(AssertionError):
        oracle.forward(q, q, np.zeros((1, 2, 1, 4), np.float32))
    with pytest.raises(ValueError):
        oracle.forward(q, q, q, order=5)
