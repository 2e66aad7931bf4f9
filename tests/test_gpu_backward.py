"""Backward pass (gdr_chunk_bwd) against the oracle's adjoint of the token loop
(oracle.backward, fp64, pinned by finite differences), on the same bf16 inputs.

Tolerance: every gradient tensor G (dq, dk, dv, d log alpha, db, dw, dS0) must satisfy
||G - G_ref||_F <= 2e-2 ||G_ref||_F.  The path rounds its matrix-core operands to bf16 (unit
roundoff 2^-8) and keeps fp32 accumulators, like the forward (whose states meet 1e-2); the
backward chains two such passes (the states, then their gradients) before the chunk-local
products and rounds its outputs to bf16, so twice the forward's state bound."""
import sys

import numpy as np
import pytest

import oracle
import synth
from gpu_util import subset_heads, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

REL = 2e-2
KINDS = {  # (alpha, b, w, shared beta): the scalar-decay family the backward covers
    "gdn": ("scalar", "scalar", "scalar", True),
    "mamba2": ("scalar", "none", "none", False),
    "deltanet": ("none", "scalar", "scalar", True),
    "la": ("none", "none", "none", False),
    "gdn_cb": ("scalar", "channel", "channel", False),
}


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


def case(kind, B=2, H=3, T=200, D=128, DV=None, s0=0.02, seed=31):
    a, b, w, shared = KINDS[kind]
    wl = synth.Workload("t", B, H, T, D, DV or D, "bf16", a, b, w, shared, -2.0, s0, seed)
    x = synth.make_prefill(wl)
    rng = np.random.default_rng(seed + 1)
    x["do"] = torch.from_numpy(rng.standard_normal((B, T, H, DV or D)).astype(np.float32)).to(torch.bfloat16)
    x["dS_T"] = torch.from_numpy((0.1 * rng.standard_normal((B, H, D, DV or D))).astype(np.float32))
    return x


def np64(t):
    return None if t is None else t.float().numpy().astype(np.float64)


def reference(x, order=0):
    return oracle.backward(np64(x["q"]), np64(x["k"]), np64(x["v"]), np64(x["log_alpha"]),
                           np64(x["b"]), np64(x["w"]), np64(x["S0"]), np64(x["do"]), np64(x["dS_T"]),
                           order=order)


def run(x, dev, order="erase_then_decay"):
    import gated_delta_rule_71_amd as gdr
    g = to_dev(x, dev)
    out = gdr.chunk_bwd(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], g["S0"], g["do"],
                        g["dS_T"], order=order)
    torch.cuda.synchronize()
    return out


def compare(out, ref, label):
    worst = 0.0
    for name in ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0"):
        r = ref[name]
        if r is None:
            assert out[name] is None, name
            continue
        got = out[name].float().cpu().numpy().astype(np.float64)
        assert got.shape == r.shape, (name, got.shape, r.shape)
        assert np.isfinite(got).all(), name
        den = np.linalg.norm(r)
        rel = float(np.linalg.norm(got - r) / den) if den > 0 else float(np.abs(got).max())
        say("  %s %-10s rel %.3e" % (label, name, rel))
        worst = max(worst, rel)
        assert rel <= REL, (label, name, rel)
    return worst


@pytest.mark.parametrize("kind", list(KINDS))
def test_backward_small(dev, kind):
    x = case(kind)
    say("backward", kind)
    compare(run(x, dev), reference(x), kind)


@pytest.mark.parametrize("D,DV", [(32, 32), (64, 48), (64, 128), (128, 16), (32, 112), (128, 256), (64, 144),
                                  (32, 192)])
def test_backward_dims(dev, D, DV):
    x = case("gdn_cb", T=133, D=D, DV=DV, seed=41)
    say("backward dims", D, DV)
    compare(run(x, dev), reference(x), "dk=%d dv=%d" % (D, DV))


def test_backward_empty_sequence(dev):
    """T = 0: no token, so dS0 = dS_T (and zeros without dS_T); the token gradients are empty."""
    x = case("gdn", B=1, H=2, T=0, seed=49)
    out = run(x, dev)
    assert out["dq"].numel() == 0 and out["dv"].numel() == 0
    np.testing.assert_array_equal(out["dS0"].cpu().numpy(), x["dS_T"].numpy())
    x["dS_T"] = None
    out = run(x, dev)
    assert not out["dS0"].abs().max().item()


@pytest.mark.parametrize("T", [1, 63, 64, 65, 128, 300])
def test_backward_lengths(dev, T):
    x = case("gdn", B=1, H=2, T=T, seed=50 + T)
    say("backward T", T)
    compare(run(x, dev), reference(x), "T=%d" % T)


def test_backward_orders_agree_under_scalar_decay(dev):
    """A scalar decay commutes with the erase: the decay-then-erase call is the same map."""
    x = case("gdn", B=1, H=2, T=150, seed=61)
    a = run(x, dev, "erase_then_decay")
    b = run(x, dev, "decay_then_erase")
    for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0"):
        assert torch.equal(a[n], b[n]), n
    compare(b, reference(x, order=1), "decay first")


def test_backward_strong_decay(dev):
    """log alpha = -7 over whole chunks (e^{G_n} ~ 1e-195 in a chunk): the chunk maps take their
    exact token path and the masks underflow to zero without overflow."""
    x = case("gdn", B=1, H=2, T=64 * 3 + 5, seed=71)
    la = x["log_alpha"].clone()
    la[:, 64:128] = -7.0
    x["log_alpha"] = la
    out = run(x, dev)
    compare(out, reference(x), "strong decay")


def test_backward_gdn_workload_sampled(dev):
    """The Gated DeltaNet workload at full size (B=4, H=16, T=4096, d=128); the oracle runs on two
    sampled (batch, head) pairs."""
    wl = synth.WORKLOADS["gdn"]
    x = synth.make_prefill(wl)
    rng = np.random.default_rng(77)
    x["do"] = torch.from_numpy(rng.standard_normal((wl.B, wl.T, wl.H, wl.DV)).astype(np.float32)).to(torch.bfloat16)
    x["dS_T"] = None
    say("backward gdn workload")
    out = run(x, dev)
    pick = [(1, 5), (3, 14)]
    bi = torch.tensor([p[0] for p in pick])
    hi = torch.tensor([p[1] for p in pick])
    xs = subset_heads({n: x[n] for n in ("q", "k", "v", "log_alpha", "b", "w", "S0", "do")}, bi, hi)
    xs["dS_T"] = None
    ref = reference(xs)
    sel = {}
    for n, t in out.items():
        if t is None:
            sel[n] = None
        elif n == "dS0":
            sel[n] = t[bi.to(t.device), hi.to(t.device)].unsqueeze(1)
        else:
            sel[n] = t[bi.to(t.device), :, hi.to(t.device)].unsqueeze(2)
    compare(sel, ref, "gdn sampled")


@pytest.mark.parametrize("kind", ["gdn", "gdn_cb"])
def test_backward_grouped_heads(dev, kind):
    """Four value heads sharing two q / k heads: dq and dk are the sums, over the value heads of a
    group, of the per-value-head gradients of the expanded problem."""
    B, H, HK, T, D = 2, 4, 2, 140, 64
    a_, b_, w_, shared = KINDS[kind]
    wl = synth.Workload("t", B, H, T, D, D, "bf16", a_, b_, w_, shared, -2.0, 0.02, 81, HK=HK)
    x = synth.make_prefill(wl)
    rng = np.random.default_rng(82)
    x["do"] = torch.from_numpy(rng.standard_normal((B, T, H, D)).astype(np.float32)).to(torch.bfloat16)
    x["dS_T"] = torch.from_numpy((0.1 * rng.standard_normal((B, H, D, D))).astype(np.float32))
    say("backward grouped", kind)
    out = run(x, dev)
    assert tuple(out["dq"].shape) == (B, T, HK, D)
    xe = synth.expand_heads({n: x[n] for n in ("q", "k", "v", "log_alpha", "b", "w", "S0")}, H)
    xe["do"], xe["dS_T"] = x["do"], x["dS_T"]
    ref = reference(xe)
    G = H // HK
    for n in ("dq", "dk"):
        ref[n] = ref[n].reshape(B, T, HK, G, D).sum(3)
    compare(out, ref, "grouped %s" % kind)


def test_backward_wide_values_grouped(dev):
    """d_v = 256 (two column halves of the chunk-local adjoint) with grouped q / k heads and
    per-channel erase and write gates: the partial sums of both kinds are added together."""
    B, H, HK, T, D, DV = 1, 4, 2, 100, 64, 256
    wl = synth.Workload("t", B, H, T, D, DV, "bf16", "scalar", "channel", "channel", False, -2.0, 0.02, 91, HK=HK)
    x = synth.make_prefill(wl)
    rng = np.random.default_rng(92)
    x["do"] = torch.from_numpy(rng.standard_normal((B, T, H, DV)).astype(np.float32)).to(torch.bfloat16)
    x["dS_T"] = torch.from_numpy((0.1 * rng.standard_normal((B, H, D, DV))).astype(np.float32))
    say("backward wide grouped")
    out = run(x, dev)
    xe = synth.expand_heads({n: x[n] for n in ("q", "k", "v", "log_alpha", "b", "w", "S0")}, H)
    xe["do"], xe["dS_T"] = x["do"], x["dS_T"]
    ref = reference(xe)
    for n in ("dq", "dk"):
        ref[n] = ref[n].reshape(B, T, HK, H // HK, D).sum(3)
    compare(out, ref, "wide grouped")
