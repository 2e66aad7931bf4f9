"""Backward pass (gdr_chunk_bwd) against the oracle's adjoint of the token loop
(oracle.backward, fp64, pinned by finite differences), on the same bf16 inputs.

Tolerance: every gradient tensor G (dq, dk, dv, d log alpha, db, dw, dS0) must satisfy
||G - G_ref||_F <= 2e-2 ||G_ref||_F, as a whole and for each (batch, head) state, and its largest
element error per state must stay within 2e-2 of that state's largest reference element.  The path rounds its matrix-core operands to bf16 (unit
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


def state_slices(name, shape):
    """Index tuples of the (batch, head) states of a gradient tensor: [B, T, H(, D)] per token,
    [B, H, dk, dv] for dS0."""
    if name == "dS0":
        return [(b, h) for b in range(shape[0]) for h in range(shape[1])]
    return [(b, slice(None), h) for b in range(shape[0]) for h in range(shape[2])]


def compare(out, ref, label, rel_tol=REL):
    """Every gradient tensor, whole and state by state: for each (batch, head) state s,
    ||G_s - G_ref,s||_F <= REL ||G_ref,s||_F and max |G_s - G_ref,s| <= REL max |G_ref,s|, so that
    an error confined to a few tokens or to one head cannot hide under the norm of the rest."""
    worst = 0.0
    for name in ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0"):
        r = ref[name]
        if r is None:
            assert out[name] is None, name
            continue
        got = out[name].float().cpu().numpy().astype(np.float64)
        assert got.shape == r.shape, (name, got.shape, r.shape)
        assert np.isfinite(got).all(), name
        if r.size == 0:
            continue
        den = np.linalg.norm(r)
        rel = float(np.linalg.norm(got - r) / den) if den > 0 else float(np.abs(got).max())
        st_f, st_m = 0.0, 0.0
        for ix in state_slices(name, r.shape):
            rs, gs = r[ix], got[ix]
            if rs.size == 0:
                continue
            nf, nm = np.linalg.norm(rs), np.abs(rs).max()
            ef, em = np.linalg.norm(gs - rs), np.abs(gs - rs).max()
            st_f = max(st_f, ef / nf if nf > 0 else ef)
            st_m = max(st_m, em / nm if nm > 0 else em)
        say("  %s %-10s rel %.3e  per state: Frobenius %.3e  max %.3e" % (label, name, rel, st_f, st_m))
        worst = max(worst, rel, st_f, st_m)
        assert rel <= rel_tol and st_f <= rel_tol and st_m <= rel_tol, (label, name, rel, st_f, st_m)
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
    """The Gated DeltaNet workload at full size (B=4, H=16, T=4096, d=128); the oracle runs on eight
    sampled (batch, head) pairs, one or two from each batch row."""
    wl = synth.WORKLOADS["gdn"]
    x = synth.make_prefill(wl)
    rng = np.random.default_rng(77)
    x["do"] = torch.from_numpy(rng.standard_normal((wl.B, wl.T, wl.H, wl.DV)).astype(np.float32)).to(torch.bfloat16)
    x["dS_T"] = None
    say("backward gdn workload")
    out = run(x, dev)
    pick = [(0, 0), (0, 9), (1, 5), (1, 15), (2, 3), (2, 12), (3, 7), (3, 14)]
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


# ---- per-channel decay (the Gated DeltaNet-2 and KDA gates), d_k = 128 ----

CH_KINDS = {  # (alpha, b, w, shared beta)
    "gdn2": ("channel", "channel", "channel", False),
    "kda": ("channel", "scalar", "scalar", True),
    "gla": ("channel", "none", "none", False),
    "gdn2_sw": ("channel", "channel", "scalar", False),
}


def ch_case(kind, B=1, H=2, T=150, DV=128, s0=0.02, seed=101, mu=-2.0):
    a, b, w, shared = CH_KINDS[kind]
    wl = synth.Workload("t", B, H, T, 128, DV, "bf16", a, b, w, shared, mu, s0, seed)
    x = synth.make_prefill(wl)
    rng = np.random.default_rng(seed + 1)
    x["do"] = torch.from_numpy(rng.standard_normal((B, T, H, DV)).astype(np.float32)).to(torch.bfloat16)
    x["dS_T"] = torch.from_numpy((0.1 * rng.standard_normal((B, H, 128, DV))).astype(np.float32))
    return x


@pytest.mark.parametrize("order", ["erase_then_decay", "decay_then_erase"])
@pytest.mark.parametrize("kind", list(CH_KINDS))
def test_backward_channel_decay(dev, kind, order):
    """Per-channel decay in either order: chunks of 64 tokens (two whole, one ragged), S0 and
    dS_T, against the token adjoint."""
    x = ch_case(kind)
    say("backward channel", kind, order)
    compare(run(x, dev, order), reference(x, order=0 if order == "erase_then_decay" else 1),
            "%s %s" % (kind, order))


@pytest.mark.parametrize("T,DV", [(1, 128), (64, 64), (65, 128), (200, 64)])
def test_backward_channel_shapes(dev, T, DV):
    x = ch_case("gdn2", T=T, DV=DV, seed=110 + T)
    say("backward channel shape", T, DV)
    compare(run(x, dev), reference(x), "T=%d dv=%d" % (T, DV))


@pytest.mark.parametrize("order", ["erase_then_decay", "decay_then_erase"])
def test_backward_channel_flagged_chunks(dev, order):
    """Chunks whose prefix sums of log alpha leave [-76, 76] take the token-by-token adjoint:
    log alpha = -7 over the second chunk on half the channels (a span of 448 nats), and -3 over
    the ragged last chunk, beside ordinary chunks."""
    x = ch_case("gdn2", T=64 * 3 + 20, seed=121)
    la = x["log_alpha"].clone()
    la[:, 64:128, :, :64] = -7.0
    la[:, 192:, :, 100:] = -3.0
    x["log_alpha"] = la
    say("backward channel flagged", order)
    compare(run(x, dev, order), reference(x, order=0 if order == "erase_then_decay" else 1),
            "flagged %s" % order)


def test_backward_channel_grouped_heads(dev):
    """KDA gates with four value heads over two q / k heads."""
    B, H, HK, T = 1, 4, 2, 130
    wl = synth.Workload("t", B, H, T, 128, 128, "bf16", "channel", "scalar", "scalar", True, -2.0, 0.02, 131,
                        HK=HK)
    x = synth.make_prefill(wl)
    rng = np.random.default_rng(132)
    x["do"] = torch.from_numpy(rng.standard_normal((B, T, H, 128)).astype(np.float32)).to(torch.bfloat16)
    x["dS_T"] = torch.from_numpy((0.1 * rng.standard_normal((B, H, 128, 128))).astype(np.float32))
    say("backward channel grouped")
    out = run(x, dev)
    xe = synth.expand_heads({n: x[n] for n in ("q", "k", "v", "log_alpha", "b", "w", "S0")}, H)
    xe["do"], xe["dS_T"] = x["do"], x["dS_T"]
    ref = reference(xe)
    for n in ("dq", "dk"):
        ref[n] = ref[n].reshape(B, T, HK, H // HK, 128).sum(3)
    compare(out, ref, "channel grouped")


@pytest.mark.parametrize("name,npick", [("kda", 8), ("gdn2", 2)])
def test_backward_channel_workload_sampled(dev, name, npick):
    """The KDA (B=2, H=32, T=8192) and Gated DeltaNet-2 (B=1, H=16, T=32768) workloads at full
    size; the oracle's adjoint (which keeps every token's state in fp64) runs on eight sampled
    (batch, head) states of KDA and two of the four times longer Gated DeltaNet-2 sequence."""
    wl = synth.WORKLOADS[name]
    x = synth.make_prefill(wl)
    rng = np.random.default_rng(141)
    x["do"] = torch.from_numpy(rng.standard_normal((wl.B, wl.T, wl.H, wl.DV)).astype(np.float32)).to(torch.bfloat16)
    x["dS_T"] = None
    say("backward channel workload", name)
    out = run(x, dev)
    pick = [(i % wl.B, (5 * i + 3) % wl.H) for i in range(npick)]
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
    compare(sel, ref, "%s sampled" % name)


@pytest.mark.parametrize("kind,order", [("gdn2", "erase_then_decay"), ("kda", "decay_then_erase"),
                                        ("gdn2_sw", "erase_then_decay")])
def test_backward_channel_same_call_same_bits(dev, kind, order):
    """The per-channel chunk-local adjoint adds its per-token and per-channel sums in a fixed
    order (no floating-point atomics), so two calls on the same inputs give the same bits."""
    x = ch_case(kind, B=2, H=3, T=64 * 3 + 9, DV=128, seed=151)
    a = run(x, dev, order)
    b = run(x, dev, order)
    for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0"):
        if a[n] is None:
            continue
        assert torch.equal(a[n], b[n]), n


@pytest.mark.parametrize("kind,DV", [("gdn", 128), ("gdn_cb", 48), ("mamba2", 256)])
def test_backward_scalar_same_call_same_bits(dev, kind, DV):
    """The scalar-decay chunk-local adjoint keeps per-wave partial sums and adds them in a fixed
    order, so two calls on the same inputs give the same bits."""
    x = case(kind, B=2, H=3, T=150, D=64 if DV == 48 else 128, DV=DV, seed=161)
    a = run(x, dev)
    b = run(x, dev)
    for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0"):
        if a[n] is None:
            continue
        assert torch.equal(a[n], b[n]), n


@pytest.mark.parametrize("kind,B,H", [("gdn", 2, 3), ("gdn", 4, 5), ("gdn", 4, 9),
                                      ("gdn2", 2, 3), ("gdn2", 4, 5), ("gdn2", 4, 9)])
def test_backward_chain_launch_forms(dev, kind, B, H):
    """The three launch forms of the state chains at d_v = 128: both chains in one launch (at most
    16 states), one after the other 16 columns wide (17 to 31 states), and 32 columns wide (32
    states and more); every state against the token adjoint."""
    if kind == "gdn":
        x = case(kind, B=B, H=H, T=64 + 7, D=128, seed=171 + H)
    else:
        x = ch_case(kind, B=B, H=H, T=64 + 7, DV=128, seed=181 + H)
    say("backward chain forms", kind, B * H, "states")
    compare(run(x, dev), reference(x), "%s %d states" % (kind, B * H))


# ---- the token adjoint: every problem outside the chunkwise backward's shapes ----

TOK_KINDS = dict(KINDS, **CH_KINDS)
REL32 = 1e-4  # all-fp32 mode: the token adjoint is fp32 throughout (the forward's fp32 bound)


def tok_case(kind, D, DV, dtype="bf16", B=1, H=2, T=37, HK=0, seed=201):
    a, b, w, shared = TOK_KINDS[kind]
    wl = synth.Workload("t", B, H, T, D, DV, dtype, a, b, w, shared, -2.0, 0.02, seed, HK=HK)
    x = synth.make_prefill(wl)
    rng = np.random.default_rng(seed + 1)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x["do"] = torch.from_numpy(rng.standard_normal((B, T, H, DV)).astype(np.float32)).to(dt)
    x["dS_T"] = torch.from_numpy((0.1 * rng.standard_normal((B, H, D, DV))).astype(np.float32))
    return x


def tok_reference(x, order, H, HK):
    if not HK or HK == H:
        return reference(x, order=order)
    xe = synth.expand_heads({n: x[n] for n in ("q", "k", "v", "log_alpha", "b", "w", "S0")}, H)
    xe["do"], xe["dS_T"] = x["do"], x["dS_T"]
    ref = reference(xe, order=order)
    B, T, _, D = x["q"].shape
    for n in ("dq", "dk"):
        ref[n] = ref[n].reshape(B, T, HK, H // HK, D).sum(3)
    return ref


@pytest.mark.parametrize("order", ["erase_then_decay", "decay_then_erase"])
@pytest.mark.parametrize("kind,D,DV", [("gdn", 16, 16), ("gdn2", 32, 48), ("kda", 64, 64), ("gdn", 128, 128),
                                       ("gdn2", 128, 256), ("gla", 256, 64), ("gdn2_sw", 256, 256),
                                       ("deltanet", 64, 32), ("la", 16, 32)])
def test_backward_fp32_mode(dev, kind, D, DV, order):
    """The all-fp32 mode at every width, both orders, against the fp64 adjoint at the fp32
    tolerance (T = 37: four whole blocks of 8 tokens and a ragged fifth)."""
    x = tok_case(kind, D, DV, "fp32", seed=211 + D + DV)
    say("backward fp32", kind, D, DV, order)
    o = 0 if order == "erase_then_decay" else 1
    compare(run(x, dev, order), reference(x, order=o), "fp32 %s %d/%d %s" % (kind, D, DV, order), rel_tol=REL32)


@pytest.mark.parametrize("kind,D,DV,order", [
    ("gdn", 256, 256, "erase_then_decay"), ("gdn2", 256, 256, "erase_then_decay"),
    ("kda", 256, 128, "decay_then_erase"), ("gdn2", 64, 64, "erase_then_decay"),
    ("kda", 32, 32, "decay_then_erase"), ("gdn2", 128, 256, "decay_then_erase"),
    ("gdn2", 16, 16, "erase_then_decay"), ("gdn_cb", 16, 64, "erase_then_decay")])
def test_backward_bf16_token_adjoint(dev, kind, D, DV, order):
    """bf16 problems outside the chunkwise backward's shapes: d_k = 256 (the width of the pages'
    Gated DeltaNet models), a per-channel decay at d_k 16, 32 and 64 or with d_v = 256, and d_k = 16
    with a scalar decay; T = 100 (twelve blocks and a ragged one)."""
    x = tok_case(kind, D, DV, "bf16", T=100, seed=231 + D + DV)
    say("backward bf16 token adjoint", kind, D, DV, order)
    o = 0 if order == "erase_then_decay" else 1
    compare(run(x, dev, order), reference(x, order=o), "bf16 tok %s %d/%d %s" % (kind, D, DV, order))


@pytest.mark.parametrize("T", [0, 1, 8, 9])
def test_backward_token_adjoint_lengths(dev, T):
    """Lengths around the 8-token blocks, T = 0 included (dS0 = dS_T and nothing else)."""
    x = tok_case("gdn2", 64, 64, "fp32", B=2, H=2, T=T, seed=251 + T)
    say("backward token adjoint T", T)
    compare(run(x, dev), reference(x), "tok T=%d" % T, rel_tol=REL32)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_backward_token_adjoint_grouped_heads(dev, dtype):
    """Four value heads over two q / k heads, d_v = 256 (two column blocks): dq and dk sum their
    value heads' parts in a fixed order."""
    B, H, HK, T = 1, 4, 2, 41
    x = tok_case("kda", 64, 256, dtype, B=B, H=H, T=T, HK=HK, seed=261)
    say("backward token adjoint grouped", dtype)
    compare(run(x, dev), tok_reference(x, 0, H, HK), "tok grouped %s" % dtype,
            rel_tol=REL if dtype == "bf16" else REL32)


def test_backward_token_adjoint_same_call_same_bits(dev):
    """Fixed-order sums: two calls on the same inputs give the same bits."""
    x = tok_case("gdn2", 256, 256, "fp32", B=1, H=2, T=29, seed=271)
    a = run(x, dev)
    b = run(x, dev)
    for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0"):
        if a[n] is not None:
            assert torch.equal(a[n], b[n]), n


def test_backward_d256_workload_sampled(dev):
    """The Gated DeltaNet gates at d_k = d_v = 256 (B=4, H=8, T=4096: the token adjoint) at full
    size; the oracle's adjoint runs on two sampled (batch, head) states."""
    wl = synth.WORKLOADS["gdn_d256"]
    x = synth.make_prefill(wl)
    rng = np.random.default_rng(281)
    x["do"] = torch.from_numpy(rng.standard_normal((wl.B, wl.T, wl.H, wl.DV)).astype(np.float32)).to(torch.bfloat16)
    x["dS_T"] = None
    say("backward d256 workload")
    out = run(x, dev)
    pick = [(1, 5), (3, 2)]
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
    compare(sel, ref, "gdn_d256 sampled")


@pytest.mark.parametrize("order", ["erase_then_decay", "decay_then_erase"])
def test_backward_token_adjoint_extreme_gates(dev, order):
    """The token adjoint has no chunk exponents to keep in range: decays of e^-60 (log alpha =
    -60 over a stretch of tokens and channels), no decay (log alpha = 0) and full erasure (b = 1)
    beside ordinary gates, in the all-fp32 mode at d_k = 64, against the fp64 adjoint."""
    x = tok_case("gdn2", 64, 64, "fp32", B=1, H=2, T=45, seed=291)
    la = x["log_alpha"].clone()
    la[:, 10:20, :, :32] = -60.0
    la[:, 30:38, :, 16:] = 0.0
    x["log_alpha"] = la
    b = x["b"].clone()
    b[:, 5:9] = 1.0
    x["b"] = b
    say("backward token adjoint extreme gates", order)
    o = 0 if order == "erase_then_decay" else 1
    compare(run(x, dev, order), reference(x, order=o), "tok extreme %s" % order, rel_tol=REL32)
