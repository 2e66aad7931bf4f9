"""State decomposition and intervention hooks ("How Linear Attention Remembers": Analytical
Framework and Causal Intervention Framework) on the HIP path, against the oracle.

Contributions C_i^(t) are compared with the definition (transition operators composed in fp64,
oracle.reference.contribution) relative to the size of the state they belong to: per (batch,
head) ||C - C_ref||_F / ||S_t||_F <= 1e-2.  Interventions are compared with oracle runs on the
same edited inputs, to the prefill tolerances (bf16 inputs: max |do| <= 2e-2, per-state
relative ||dS||_F <= 1e-2).
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from gpu_util import TOL, errors, to_dev
from oracle import reference as ref

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_71_amd as gdr
    gdr._native.lib()  # fails loudly if the library is not built
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


KINDS = {"gdn2": ("channel", "channel", "channel", False), "gdn": ("scalar", "scalar", "scalar", True),
         "kda": ("channel", "scalar", "scalar", True)}


def inputs(kind, B=2, H=3, T=200, D=64, seed=5, s0=0.0):
    a, b, w, shared = KINDS[kind]
    wl = synth.Workload("h", B, H, T, D, D, "bf16", a, b, w, shared, -2.0, s0, seed)
    return synth.make_prefill(wl)


def np64(x):
    return None if x is None else x.float().numpy().astype(np.float64)


def args(x):
    return (x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"])


@pytest.mark.parametrize("kind", list(KINDS))
def test_contributions_match_the_definition_and_sum_to_the_state(dev, kind):
    from gated_delta_rule_71_amd import hooks, chunk_fwd
    x = inputs(kind)
    g = to_dev(x, dev)
    t, pos = 199, [0, 37, 63, 64, 130, 199]
    say("contributions", kind, pos, "t =", t)
    C = hooks.contributions(*args(g), positions=pos, t=t).cpu().numpy().astype(np.float64)
    xa = [np64(a) for a in args(x)]
    _, S_ref = oracle.forward(*args(x), None)
    scale = np.linalg.norm(S_ref.reshape(S_ref.shape[0], S_ref.shape[1], -1), axis=-1)
    worst = 0.0
    for j, i in enumerate(pos):
        Cr = ref.contribution(*xa, i=i, t=t)
        d = np.linalg.norm((C[j] - Cr).reshape(Cr.shape[0], Cr.shape[1], -1), axis=-1)
        worst = max(worst, float((d / scale).max()))
    say("  max ||dC|| / ||S_t|| = %.3e" % worst)
    assert worst <= 1e-2
    # every position at once: the kernel's contributions add up to the kernel's own S_t
    Call = hooks.contributions(*args(g), positions=range(t + 1), t=t).sum(0)
    _, S = chunk_fwd(*args(g), None)
    rel = (torch.linalg.vector_norm((Call - S).flatten(2), dim=-1) /
           torch.linalg.vector_norm(S.flatten(2), dim=-1)).max().item()
    say("  ||sum_i C_i - S_t|| / ||S_t|| = %.3e" % rel)
    assert rel <= 1e-2


@pytest.mark.parametrize("kind", ["gdn2", "gdn"])
def test_block_write(dev, kind):
    from gated_delta_rule_71_amd import hooks
    x = inputs(kind, s0=0.02)
    g = to_dev(x, dev)
    pos = 77
    o, S = hooks.block_write(*args(g), S0=g["S0"], position=pos)
    torch.cuda.synchronize()
    w = x["w"].clone()
    w[:, pos] = 0
    o_ref, S_ref = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], w, x["S0"])
    eo, es = errors(o, S, o_ref, S_ref)
    say("block_write %s: max|do|=%.3e rel|dS|=%.3e" % (kind, eo, es))
    assert eo <= TOL["bf16"][0] and es <= TOL["bf16"][1]


def test_replace_write(dev):
    from gated_delta_rule_71_amd import hooks
    x = inputs("gdn2", s0=0.02)
    dn = inputs("gdn2", seed=9)
    g, gd = to_dev(x, dev), to_dev(dn, dev)
    pos = 120
    o, S = hooks.replace_write(*args(g), S0=g["S0"], position=pos,
                               donor={"k": gd["k"], "v": gd["v"], "w": gd["w"]})
    torch.cuda.synchronize()
    # the definition: S_t - C_x^(t) + (T_t o ... o T_{x+1})(k'_x^T (w'_x . v'_x))
    w0 = x["w"].clone()
    w0[:, pos] = 0
    o1, S1 = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], w0, x["S0"])
    kd = np64(dn["k"])[:, pos]
    xd = np64(dn["w"])[:, pos] * np64(dn["v"])[:, pos]
    S2 = ref.contribution(*[np64(a) for a in args(x)], i=pos, write=(kd, xd))
    # the read-out of the donor write, tokens pos.. (an oracle run holding only that write)
    k2, v2, w2 = x["k"].clone(), x["v"].clone(), torch.zeros_like(x["w"])
    k2[:, pos], v2[:, pos], w2[:, pos] = dn["k"][:, pos], dn["v"][:, pos], dn["w"][:, pos]
    o2, S2b = oracle.forward(x["q"], k2, v2, x["log_alpha"], x["b"], w2, None)
    np.testing.assert_allclose(S2b, S2, rtol=1e-9, atol=1e-12)  # the oracle agrees with itself
    eo, es = errors(o, S, o1 + o2, S1 + S2)
    say("replace_write: max|do|=%.3e rel|dS|=%.3e" % (eo, es))
    assert eo <= TOL["bf16"][0] and es <= TOL["bf16"][1]


def test_swap_state(dev):
    from gated_delta_rule_71_amd import hooks
    x = inputs("kda", s0=0.02)
    dn = inputs("kda", seed=11)
    g, gd = to_dev(x, dev), to_dev(dn, dev)
    pos = 140
    o, S, S_rec, S_don = hooks.swap_state(*args(g), S0=g["S0"], position=pos,
                                          donor={n: gd[n] for n in ("q", "k", "v", "log_alpha", "b", "w")})
    torch.cuda.synchronize()
    p = pos + 1
    head = lambda a: None if a is None else a[:, :p]
    tail = lambda a: None if a is None else a[:, p:]
    _, Sd = oracle.forward(*[head(a) for a in args(dn)], x["S0"])
    _, Sr = oracle.forward(*[head(a) for a in args(x)], x["S0"])
    o_ref, S_ref = oracle.forward(*[tail(a) for a in args(x)], Sd)
    eo, es = errors(o, S, o_ref, S_ref)
    _, er = errors(o[:, :0], S_rec, o_ref[:, :0], Sr)
    _, ed = errors(o[:, :0], S_don, o_ref[:, :0], Sd)
    say("swap_state: max|do|=%.3e rel|dS|=%.3e (pre-swap states %.2e, %.2e)" % (eo, es, er, ed))
    assert eo <= TOL["bf16"][0] and max(es, er, ed) <= TOL["bf16"][1]
