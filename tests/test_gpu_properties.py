"""Properties of the recurrence that the HIP path must keep, on the GPU, through the C ABI.

- Resume: S_t depends only on S_{t-1} and token t ("How Linear Attention Remembers", Analytical
  Framework: S_t = T_t(S_{t-1}) + W_t).  A prefill split at any token, the second call starting
  from the first one's final state, equals one call over the whole sequence; a prefill of T tokens
  followed by N decode steps equals a prefill of T + N tokens.
- Column independence: the transition multiplies S from the left ("Recurrent Memory: Write,
  Erase, Decay, Read", section 05), so each value column of S and o evolves on its own.
  Permuting the columns of v (and of a per-channel write gate) and of S0 permutes those of o and
  S_T; a state's result does not depend on how many other states share the call beyond rounding
  (bit for bit where only the column slicing of a per-state kernel changes).
- Determinism: the same call twice gives the same bits.
- In place: S_T may be S0 (the header promises it) on every kernel family.
- Parity at the shapes added to the boundary: the all-fp32 mode at d_k = 64, 128 and 256, bf16
  at d_k = 256 with the per-channel decay after the erase, and chunks whose gates span past the
  chunk form's range through the all-modes kernel (fp32 at d_k 16 and 32, bf16 at d_k 16, and d_k
  256 with the decay first).
Tolerances: max |o - o_ref| <= 2e-2 and per-state relative Frobenius ||S_T - S_ref|| <= 1e-2 with
bf16 inputs; 1e-4 in the all-fp32 mode.
"""
import sys

import numpy as np
import pytest

import synth
from gpu_util import TOL, errors, run_oracle, to_dev

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


KINDS = {  # (alpha, b, w, shared beta)
    "gdn": ("scalar", "scalar", "scalar", True),
    "kda": ("channel", "scalar", "scalar", True),
    "gdn2": ("channel", "channel", "channel", False),
    "la": ("none", "none", "none", False),
    "gla": ("channel", "none", "channel", False),
}


def case(kind, B=2, H=3, T=200, D=128, DV=None, dtype="bf16", s0=0.02, seed=7):
    a, b, w, shared = KINDS[kind]
    return synth.Workload("t", B, H, T, D, DV or D, dtype, a, b, w, shared, -2.0, s0, seed)


def fwd(g, order="erase_then_decay", S0="given", **kw):
    import gated_delta_rule_71_amd as gdr
    return gdr.chunk_fwd(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"],
                         g["S0"] if S0 == "given" else S0, order=order, **kw)


def check(x, o, S, order, tol, label):
    o_ref, S_ref = run_oracle(x, 0 if order == "erase_then_decay" else 1)
    eo, es = errors(o, S, o_ref, S_ref)
    say("%s: max|do|=%.3e rel|dS|=%.3e" % (label, eo, es))
    assert eo <= tol[0] and es <= tol[1], (label, eo, es)


def tokens(x, lo, hi):
    return {n: (None if t is None or n == "S0" else t[:, lo:hi].contiguous()) for n, t in x.items()}


def max_diff(a, b):
    return (a.float() - b.float()).abs().max().item() if a.numel() else 0.0


# ------------------------------------------------------------------ resume


@pytest.mark.parametrize("kind,T,split", [("gdn", 2100, 1000), ("gdn2", 2100, 1000), ("kda", 700, 64),
                                          ("gla", 500, 321), ("gdn2", 300, 1)])
def test_prefill_resumes_from_its_final_state(dev, kind, T, split):
    """Two calls split at `split` (not a multiple of the chunk, except 64) against one call and
    against the oracle: the split point moves every later chunk boundary, so the two runs round
    differently but both meet the tolerance."""
    wl = case(kind, B=1, H=2, T=T, seed=201)
    x = synth.make_prefill(wl)
    g = to_dev(x, dev)
    o_all, S_all = fwd(g)
    a, b = tokens(g, 0, split), tokens(g, split, T)
    o1, S1 = fwd(a, S0=g["S0"])
    o2, S2 = fwd(b, S0=S1)
    torch.cuda.synchronize()
    o_cat = torch.cat([o1, o2], 1)
    say("resume %s split %d: max|o_split - o_one| = %.3e" % (kind, split, max_diff(o_cat, o_all)))
    check(x, o_cat, S2, "erase_then_decay", TOL["bf16"], "resume %s split %d" % (kind, split))
    check(x, o_all, S_all, "erase_then_decay", TOL["bf16"], "one call %s" % kind)


@pytest.mark.parametrize("kind,D,dtype", [("gdn2", 128, "bf16"), ("gdn", 64, "bf16"), ("kda", 32, "fp32")])
def test_prefill_then_decode_equals_longer_prefill(dev, kind, D, dtype):
    """Prefill T tokens, then decode N more one at a time from its final state, against one
    prefill of all T + N tokens."""
    import gated_delta_rule_71_amd as gdr
    T, N = 190, 7
    wl = case(kind, B=2, H=2, T=T + N, D=D, dtype=dtype, seed=211)
    x = synth.make_prefill(wl)
    g = to_dev(x, dev)
    o_all, S_all = fwd(g)
    o_pre, S = fwd(tokens(g, 0, T), S0=g["S0"])
    outs = [o_pre]
    for t in range(T, T + N):
        s = tokens(g, t, t + 1)
        outs.append(gdr.decode_step(s["q"], s["k"], s["v"], s["log_alpha"], s["b"], s["w"], S))
    torch.cuda.synchronize()
    o_cat = torch.cat(outs, 1)
    say("prefill + decode %s: max|o - o_one| = %.3e" % (kind, max_diff(o_cat, o_all)))
    check(x, o_cat, S, "erase_then_decay", TOL[dtype], "prefill+decode %s" % kind)
    check(x, o_all, S_all, "erase_then_decay", TOL[dtype], "prefill %s" % kind)


# ------------------------------------------------------------------ determinism, columns


@pytest.mark.parametrize("kind,D,DV,dtype", [("gdn", 128, 128, "bf16"), ("gdn2", 128, 128, "bf16"),
                                             ("kda", 64, 64, "bf16"), ("gla", 128, 128, "bf16"),
                                             ("gdn2", 128, 128, "fp32"), ("gdn2", 256, 128, "bf16")])
def test_same_call_same_bits(dev, kind, D, DV, dtype):
    wl = case(kind, B=2, H=3, T=333, D=D, DV=DV, dtype=dtype, seed=221)
    g = to_dev(synth.make_prefill(wl), dev)
    o1, S1 = fwd(g)
    o2, S2 = fwd(g)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("kind,D,segmented", [("gdn", 128, True), ("gdn2", 128, True), ("kda", 128, True),
                                               ("gla", 128, False), ("gdn2", 64, False), ("kda", 32, False)])
def test_state_result_among_other_states(dev, kind, D, segmented):
    """Two states alone, then the same two as the first heads of a 64-state call.  Where the
    column slicing of a per-state kernel changes with the number of states, every column still
    follows the same arithmetic, so the bits agree.  The fused segment kernel (d_k = d_v = 128 with
    the Gated DeltaNet, KDA and Gated DeltaNet-2 gates) splits each sequence into more segments
    when there are fewer states, which moves rounding: there the two results agree within the
    tolerance, and both meet it against the oracle."""
    small = case(kind, B=1, H=2, T=300, D=D, seed=231)
    big = case(kind, B=1, H=64, T=300, D=D, seed=232)
    xs, xb = synth.make_prefill(small), synth.make_prefill(big)
    for n in xs:
        if xs[n] is None:
            continue
        if n == "S0":
            xb[n][:, :2] = xs[n]
        else:
            xb[n][:, :, :2] = xs[n]
    gs, gb = to_dev(xs, dev), to_dev(xb, dev)
    o_s, S_s = fwd(gs)
    o_b, S_b = fwd(gb)
    torch.cuda.synchronize()
    d_o, d_s = max_diff(o_s, o_b[:, :, :2]), max_diff(S_s, S_b[:, :2])
    say("%s d%d: 2 states alone vs among 64: max|do| = %.3e max|dS| = %.3e" % (kind, D, d_o, d_s))
    if not segmented:
        assert d_o == 0.0 and d_s == 0.0
    else:
        check(xs, o_s, S_s, "erase_then_decay", TOL["bf16"], "%s alone" % kind)
        check(xs, o_b[:, :, :2], S_b[:, :2], "erase_then_decay", TOL["bf16"], "%s among 64" % kind)
        assert d_o <= TOL["bf16"][0]


@pytest.mark.parametrize("kind,dtype", [("gdn", "bf16"), ("gdn2", "bf16"), ("gla", "bf16"), ("gdn2", "fp32")])
def test_value_columns_permute(dev, kind, dtype):
    """Permuting the value columns (v, a per-channel w and the columns of S0) permutes the columns
    of o and S_T.  A column lands in another lane of the matrix-core tiles, whose per-element
    arithmetic is the same, so the results agree to the last bit or nearly."""
    wl = case(kind, B=1, H=2, T=260, D=64 if dtype == "fp32" else 128, dtype=dtype, seed=241)
    x = synth.make_prefill(wl)
    perm = torch.from_numpy(np.random.default_rng(242).permutation(wl.DV))
    xp = dict(x)
    xp["v"] = x["v"][..., perm].contiguous()
    if x["w"] is not None and x["w"].dim() == 4:
        xp["w"] = x["w"][..., perm].contiguous()
    xp["S0"] = x["S0"][..., perm].contiguous()
    o, S = fwd(to_dev(x, dev))
    op, Sp = fwd(to_dev(xp, dev))
    torch.cuda.synchronize()
    pd = perm.to(dev)
    d_o, d_s = max_diff(o[..., pd], op), max_diff(S[..., pd], Sp)
    say("%s %s permuted columns: max|do| = %.3e max|dS| = %.3e" % (kind, dtype, d_o, d_s))
    assert d_o <= 1e-6 * max(1.0, o.float().abs().max().item())
    assert d_s <= 1e-6 * max(1.0, S.abs().max().item())


# ------------------------------------------------------------------ in place


@pytest.mark.parametrize("kind,D,DV,dtype", [("gdn", 128, 128, "bf16"), ("gdn2", 128, 128, "bf16"),
                                             ("gla", 128, 128, "bf16"), ("gdn2", 32, 48, "fp32"),
                                             ("gdn2", 128, 64, "fp32"), ("gdn", 16, 32, "bf16"),
                                             ("gdn2", 256, 64, "bf16")])
def test_final_state_in_place(dev, kind, D, DV, dtype):
    """final_state = S0: every kernel family reads S0 before it writes the final state."""
    wl = case(kind, B=2, H=2, T=150, D=D, DV=DV, dtype=dtype, seed=251)
    x = synth.make_prefill(wl)
    g = to_dev(x, dev)
    o_ref, S_ref = fwd(g)
    S = g["S0"].clone()
    o, S_out = fwd(g, S0=S, final_state=S)
    torch.cuda.synchronize()
    assert S_out.data_ptr() == S.data_ptr()
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    check(x, o, S, "erase_then_decay", TOL[dtype], "in place %s d%d/%d %s" % (kind, D, DV, dtype))


# ------------------------------------------------------------------ shapes added to the boundary


@pytest.mark.parametrize("D,DV", [(64, 64), (128, 128), (128, 48), (256, 256), (256, 32)])
@pytest.mark.parametrize("kind", ["gdn", "gdn2", "kda", "la"])
@pytest.mark.parametrize("order", ["erase_then_decay", "decay_then_erase"])
def test_prefill_fp32_wide(dev, D, DV, kind, order):
    """The all-fp32 mode at d_k = 64, 128 and 256, against the oracle at 1e-4."""
    wl = case(kind, B=1, H=2, T=150, D=D, DV=DV, dtype="fp32", seed=261)
    x = synth.make_prefill(wl)
    say("fp32", kind, D, DV, order)
    o, S = fwd(to_dev(x, dev), order=order)
    torch.cuda.synchronize()
    check(x, o, S, order, TOL["fp32"], "fp32 %s d%d/%d %s" % (kind, D, DV, order))


@pytest.mark.parametrize("kind,DV", [("gdn2", 256), ("kda", 64), ("gdn2", 48)])
def test_prefill_dk256_erase_first_channel(dev, kind, DV):
    """bf16 at d_k = 256 with a per-channel decay after the erase (the unified equation's order)."""
    wl = case(kind, B=1, H=2, T=140, D=256, DV=DV, seed=271)
    x = synth.make_prefill(wl)
    say("dk256 erase first", kind, DV)
    o, S = fwd(to_dev(x, dev))
    torch.cuda.synchronize()
    check(x, o, S, "erase_then_decay", TOL["bf16"], "dk256 %s dv%d" % (kind, DV))


def flagged(x, chunks):
    la = x["log_alpha"].clone()
    for c in chunks:
        la[:, 64 * c:64 * (c + 1)] = -7.0
    x = dict(x)
    x["log_alpha"] = la
    return x


@pytest.mark.parametrize("kind,D,DV,dtype,order", [
    ("gdn2", 16, 32, "fp32", "erase_then_decay"), ("kda", 32, 32, "fp32", "erase_then_decay"),
    ("gdn2", 32, 48, "fp32", "decay_then_erase"), ("gdn2", 16, 16, "bf16", "erase_then_decay"),
    ("kda", 16, 48, "bf16", "decay_then_erase"), ("kda", 256, 64, "bf16", "decay_then_erase"),
    ("gla", 16, 32, "fp32", "erase_then_decay")])
def test_flagged_chunks_in_the_all_modes_kernel(dev, kind, D, DV, dtype, order):
    """log alpha = -7 over whole chunks (448 nats per chunk, past the split factors' range), next
    to ordinary chunks and in the ragged last chunk, through the all-modes kernel's exact token
    path: the fp32 mode, bf16 at d_k = 16, and d_k = 256 with the decay first."""
    wl = case(kind, B=1, H=2, T=64 * 4 + 23, D=D, DV=DV, dtype=dtype, seed=281)
    x = flagged(synth.make_prefill(wl), (1, 2, 4))
    say("flagged all-modes", kind, D, DV, dtype, order)
    o, S = fwd(to_dev(x, dev), order=order)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    check(x, o, S, order, TOL[dtype], "flagged %s d%d/%d %s %s" % (kind, D, DV, dtype, order))


def test_mfma_probe_exact_result(dev):
    """The calibration probe's documented result: every operand element is 1/16, so each of a
    wave's 8 x 4 accumulator elements gains 32/256 per step and their sum is 4 * iters."""
    import gated_delta_rule_71_amd as gdr
    say("mfma probe")
    out, flop = gdr.mfma_probe(300, 6, dev)
    torch.cuda.synchronize()
    assert out.shape == (48,)
    assert bool((out == 1200.0).all())
    assert flop == 300 * 6 * 8 * 8 * 2 * 16 * 16 * 32
