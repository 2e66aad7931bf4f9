"""Parity of the HIP path (through the C ABI) against the fp64 oracle on the same seeded inputs.

Small cases span several 64-token chunks and a ragged tail; the full-size workloads are checked
on every output for the tiny and Gated DeltaNet workloads and on sampled (batch, head) states for
the larger ones.  Tolerances: max |o - o_ref| <= 2e-2 and per-state ||S_T - S_ref||_F /
||S_ref||_F <= 1e-2 with bf16 inputs; 1e-4 for both in the all-fp32 mode.
"""
import sys

import numpy as np
import pytest

import synth
from gpu_util import TOL, errors, run_gpu_prefill, run_oracle, subset_heads, workload

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
    "deltanet": ("none", "scalar", "scalar", True),
    "mamba2": ("scalar", "none", "none", False),
}


def case(kind, B=2, H=3, T=200, D=128, DV=None, dtype="bf16", s0=0.02, seed=7):
    a, b, w, shared = KINDS[kind]
    return synth.Workload("t", B, H, T, D, DV or D, dtype, a, b, w, shared, -2.0, s0, seed)


def check(x, o, S, order, tol, label):
    o_ref, S_ref = run_oracle(x, 0 if order == "erase_then_decay" else 1)
    eo, es = errors(o, S, o_ref, S_ref)
    say("%s: max|do|=%.3e rel|dS|=%.3e" % (label, eo, es))
    assert eo <= tol[0] and es <= tol[1], (label, eo, es)


@pytest.mark.parametrize("kind", list(KINDS))
@pytest.mark.parametrize("order", ["erase_then_decay", "decay_then_erase"])
def test_prefill_small_bf16(dev, kind, order):
    wl = case(kind, T=200)
    say("prefill", kind, order, wl)
    x = synth.make_prefill(wl)
    o, S = run_gpu_prefill(x, dev, order)
    torch.cuda.synchronize()
    check(x, o, S, order, TOL["bf16"], "prefill %s %s" % (kind, order))


@pytest.mark.parametrize("D", [16, 32, 64])
@pytest.mark.parametrize("kind", ["gdn", "gdn2", "kda"])
def test_prefill_small_dims_bf16(dev, D, kind):
    for DV in sorted({16, D, 2 * D if 2 * D <= 256 else D}):
        wl = case(kind, T=133, D=D, DV=DV)
        say("prefill dims", kind, D, DV)
        x = synth.make_prefill(wl)
        o, S = run_gpu_prefill(x, dev)
        torch.cuda.synchronize()
        check(x, o, S, "erase_then_decay", TOL["bf16"], "dims %s dk=%d dv=%d" % (kind, D, DV))


@pytest.mark.parametrize("D", [16, 32])
@pytest.mark.parametrize("kind", ["gdn", "gdn2", "kda", "la"])
def test_prefill_fp32_mode(dev, D, kind):
    wl = case(kind, T=150, D=D, dtype="fp32")
    say("prefill fp32", kind, D)
    x = synth.make_prefill(wl)
    o, S = run_gpu_prefill(x, dev)
    torch.cuda.synchronize()
    check(x, o, S, "erase_then_decay", TOL["fp32"], "fp32 %s dk=%d" % (kind, D))


def test_tiny_workload_fp32(dev):
    wl = synth.WORKLOADS["tiny"]
    say("tiny workload", wl)
    x = synth.make_prefill(wl)
    o, S = run_gpu_prefill(x, dev)
    torch.cuda.synchronize()
    check(x, o, S, "erase_then_decay", TOL["fp32"], "tiny")


@pytest.mark.parametrize("T", [0, 1, 63, 64, 65, 128])
def test_prefill_edge_lengths(dev, T):
    wl = case("gdn2", B=1, H=2, T=T)
    say("edge T", T)
    x = synth.make_prefill(wl)
    o, S = run_gpu_prefill(x, dev)
    torch.cuda.synchronize()
    if T == 0:
        np.testing.assert_array_equal(S.cpu().numpy(), x["S0"].numpy())
        return
    check(x, o, S, "erase_then_decay", TOL["bf16"], "T=%d" % T)


def test_prefill_extreme_gates(dev):
    wl = case("gdn2", B=1, H=2, T=160)
    x = synth.make_prefill(wl)
    x["log_alpha"] = torch.full_like(x["log_alpha"], -7.0)
    x["b"] = torch.ones_like(x["b"])
    x["w"] = torch.ones_like(x["w"])
    say("extreme channel gates")
    o, S = run_gpu_prefill(x, dev)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    check(x, o, S, "erase_then_decay", TOL["bf16"], "extreme channel")
    wl = case("gdn", B=1, H=2, T=160)
    x = synth.make_prefill(wl)
    x["log_alpha"] = torch.full_like(x["log_alpha"], -20.0)
    x["b"] = torch.ones_like(x["b"])
    x["w"] = x["b"]
    say("extreme scalar gates")
    o, S = run_gpu_prefill(x, dev)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    check(x, o, S, "erase_then_decay", TOL["bf16"], "extreme scalar")


@pytest.mark.parametrize("order", ["erase_then_decay", "decay_then_erase"])
@pytest.mark.parametrize("kind,DV", [("gdn2", 128), ("kda", 128), ("kda", 48), ("gla", 128), ("gla", 48)])
def test_prefill_flagged_chunks_mixed(dev, kind, DV, order):
    """Chunks whose per-channel gate prefix sums span past the range of the chunk form (log alpha
    = -7 over a chunk spans 448 nats) run token by token.  Here they sit between ordinary chunks
    of the same state, past the 64th chunk, and in the ragged last chunk."""
    T = 64 * 66 + 17
    wl = case(kind, B=1, H=2, T=T, DV=DV)
    x = synth.make_prefill(wl)
    la = x["log_alpha"].clone()
    for c in (1, 2, 40, 65, 66):
        la[:, 64 * c:64 * (c + 1)] = -7.0
    x["log_alpha"] = la
    say("flagged chunks", kind, "dv", DV, order)
    o, S = run_gpu_prefill(x, dev, order=order)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    check(x, o, S, order, TOL["bf16"], "flagged %s dv=%d %s" % (kind, DV, order))


@pytest.mark.parametrize("order", ["erase_then_decay", "decay_then_erase"])
@pytest.mark.parametrize("B,H,DV", [(8, 16, 128), (4, 16, 256)])
@pytest.mark.parametrize("kind", ["gdn2", "gla"])
def test_prefill_channel_wide_slices(dev, kind, B, H, DV, order):
    """Enough states that every workgroup of the per-channel state kernel takes a 64-column slice
    (states x d_v / 64 >= 256), with d_v = 256 taking the wide chunk-local kernel too."""
    wl = case(kind, B=B, H=H, T=130, D=128, DV=DV, seed=21)
    x = synth.make_prefill(wl)
    say("wide slices", kind, B, H, DV, order)
    o, S = run_gpu_prefill(x, dev, order=order)
    torch.cuda.synchronize()
    check(x, o, S, order, TOL["bf16"], "wide slices %s B=%d H=%d dv=%d %s" % (kind, B, H, DV, order))


@pytest.mark.parametrize("order", ["erase_then_decay", "decay_then_erase"])
@pytest.mark.parametrize("D", [32, 64])
@pytest.mark.parametrize("kind", ["kda", "gla"])
def test_prefill_flagged_chunks_small_dk(dev, kind, D, order):
    """Flagged chunks (log alpha = -7 over a chunk) at d_k = 32 and 64, next to ordinary ones."""
    wl = case(kind, B=1, H=2, T=64 * 3 + 9, D=D, seed=23)
    x = synth.make_prefill(wl)
    la = x["log_alpha"].clone()
    la[:, 64:128] = -7.0
    la[:, 192:] = -7.0
    x["log_alpha"] = la
    say("flagged chunks dk", kind, D, order)
    o, S = run_gpu_prefill(x, dev, order=order)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    check(x, o, S, order, TOL["bf16"], "flagged %s dk=%d %s" % (kind, D, order))


# ------------------------------------------------------------------ decode


@pytest.mark.parametrize("kind", list(KINDS))
@pytest.mark.parametrize("order", ["erase_then_decay", "decay_then_erase"])
@pytest.mark.parametrize("D,DV,dtype", [(128, 128, "bf16"), (64, 32, "bf16"), (16, 48, "fp32"),
                                        (32, 64, "fp32")])
def test_decode_steps(dev, kind, order, D, DV, dtype):
    import gated_delta_rule_71_amd as gdr
    wl = case(kind, B=3, H=2, T=1, D=D, DV=DV, dtype=dtype)
    say("decode", kind, order, D, DV, dtype)
    S_host = None
    S = None
    for step in range(3):
        x = synth.make_prefill(wl, seed=100 + step)
        if S is None:
            S = x["S0"].to(dev)
            S_host = x["S0"].double().numpy()
        g = {n: (None if t is None else t.to(dev)) for n, t in x.items()}
        o = gdr.decode_step(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], S, order=order)
        x = dict(x)
        x["S0"] = S_host
        o_ref, S_host = run_oracle(x, 0 if order == "erase_then_decay" else 1)
        torch.cuda.synchronize()
        tol = TOL[dtype]
        eo, es = errors(o, S, o_ref, S_host)
        assert eo <= tol[0] and es <= tol[1], (step, eo, es)
    say("decode ok", eo, es)


def test_decode_workload_subset(dev):
    """The decode workload at full size (256 x 32 states, 537 MB) for 1000 steps; the oracle
    follows 64 seeded states across every step."""
    import gated_delta_rule_71_amd as gdr
    wl = synth.WORKLOADS["decode"]
    n_steps = wl.steps
    say("decode workload", wl)
    S = synth.make_decode_state(wl, dev)
    steps = synth.make_decode_steps(wl, n_steps, dev)
    rng = np.random.default_rng(5)
    pick = rng.choice(wl.B * wl.H, size=64, replace=False)
    bi = torch.tensor(pick // wl.H, device=dev)
    hi = torch.tensor(pick % wl.H, device=dev)
    S_host = S[bi, hi].double().cpu().numpy()[:, None]          # [64, 1, DK, DV]
    sub = {n: (None if t is None else t[:, bi, 0, hi].cpu()) for n, t in steps.items()}
    o_sel = []
    for i in range(n_steps):
        t = {n: (None if v is None else v[i]) for n, v in steps.items()}
        o = gdr.decode_step(t["q"], t["k"], t["v"], t["log_alpha"], t["b"], t["w"], S)
        o_sel.append(o[bi, 0, hi])
    o_sel = torch.stack(o_sel).float().cpu().numpy()            # [n, 64, DV]
    S_fin = S[bi, hi].double().cpu().numpy()
    say("decode workload: GPU done")
    worst_o = 0.0
    for i in range(n_steps):
        x = {}
        for n, v in sub.items():
            x[n] = None if v is None else v[i].reshape((64, 1, 1) + tuple(v.shape[2:]))
        x["S0"] = S_host
        o_ref, S_host = run_oracle(x)
        worst_o = max(worst_o, float(np.abs(o_sel[i][:, None, None] - o_ref).max()))
    rel = (np.linalg.norm((S_fin - S_host[:, 0]).reshape(64, -1), axis=1)
           / np.linalg.norm(S_host[:, 0].reshape(64, -1), axis=1)).max()
    say("decode workload: max|do|=%.3e  rel|dS|=%.3e" % (worst_o, rel))
    assert worst_o <= 2e-2 and rel <= 1e-2


# ------------------------------------------------------------------ full-size prefill workloads


@pytest.mark.parametrize("name", ["gdn", "mamba2", "gdn_gqa"])
def test_scalar_decay_workloads_full(dev, name):
    wl = synth.WORKLOADS[name]
    say("%s workload" % name, wl)
    x = synth.make_prefill(wl)
    o, S = run_gpu_prefill(x, dev)
    torch.cuda.synchronize()
    check(synth.expand_heads(x, wl.H), o, S, "erase_then_decay", TOL["bf16"], "%s full" % name)


@pytest.mark.parametrize("name", ["kda", "gdn2", "gla", "gdn_d256"])
def test_large_workloads_sampled(dev, name):
    """The per-channel workloads and the d_k = 256 one at full size, eight states checked."""
    wl = synth.WORKLOADS[name]
    say("%s workload (sampled states)" % name, wl)
    x = synth.make_prefill(wl)
    o, S = run_gpu_prefill(x, dev)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    n = min(8, wl.B * wl.H)
    pick = rng.choice(wl.B * wl.H, size=n, replace=False)
    bi, hi = torch.tensor(pick // wl.H), torch.tensor(pick % wl.H)
    xs = subset_heads(x, bi, hi)
    o_ref, S_ref = run_oracle(xs)
    o_sel = o[bi.to(dev), :, hi.to(dev)].unsqueeze(2)
    S_sel = S[bi.to(dev), hi.to(dev)].unsqueeze(1)
    eo, es = errors(o_sel, S_sel, o_ref, S_ref)
    say("%s sampled: max|do|=%.3e rel|dS|=%.3e" % (name, eo, es))
    assert eo <= TOL["bf16"][0] and es <= TOL["bf16"][1]


# ------------------------------------------------------------------ the timing-marker entry point


@pytest.mark.parametrize("kind,dtype", [("gdn", "bf16"), ("gdn2", "bf16"), ("kda", "fp32")])
def test_marked_call_matches_plain_call(dev, kind, dtype):
    """gdr_chunk_fwd_marked runs the same kernels as gdr_chunk_fwd (identical bits) and records
    its event between the start and the end of the call."""
    import gated_delta_rule_71_amd as gdr
    from gpu_util import to_dev
    wl = case(kind, T=200, D=64 if dtype == "bf16" else 32, dtype=dtype)
    say("marked", kind, dtype, wl)
    g = to_dev(synth.make_prefill(wl), dev)
    args = (g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], g["S0"])
    o1, S1 = gdr.chunk_fwd(*args)
    stream = torch.cuda.current_stream(dev)
    e0, em, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e0.record(stream)
    o2, S2 = gdr.chunk_fwd(*args, phase_event=em)
    e1.record(stream)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    t_a, t_b = e0.elapsed_time(em), em.elapsed_time(e1)
    say("phases: %.4f ms + %.4f ms" % (t_a, t_b))
    assert t_a >= 0.0 and t_b > 0.0
    x = synth.make_prefill(wl)
    check(x, o2, S2, "erase_then_decay", TOL[dtype], "marked %s %s" % (kind, dtype))


# ------------------------------------------------------------------ grouped key / value heads


def grouped(x, G):
    """Inputs whose q and k have H / G heads (value head h reads q / k head h // G): the kernel's
    copy keeps every G-th q / k head, the oracle's repeats those G times."""
    xq = dict(x)
    for n in ("q", "k"):
        xq[n] = x[n][:, :, ::G].contiguous()
    xr = dict(x)
    for n in ("q", "k"):
        xr[n] = xq[n].repeat_interleave(G, dim=2)
    return xq, xr


@pytest.mark.parametrize("kind,D,dtype", [("gdn", 128, "bf16"), ("kda", 64, "bf16"), ("gdn2", 128, "bf16"),
                                          ("mamba2", 64, "bf16"), ("gdn", 16, "bf16"), ("gdn2", 32, "fp32")])
def test_prefill_grouped_heads(dev, kind, D, dtype):
    import gated_delta_rule_71_amd as gdr
    from gpu_util import to_dev
    wl = case(kind, B=2, H=4, T=200, D=D, dtype=dtype)
    say("grouped heads", kind, D, dtype)
    xq, xr = grouped(synth.make_prefill(wl), 2)
    g = to_dev(xq, dev)
    o, S = gdr.chunk_fwd(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], g["S0"])
    torch.cuda.synchronize()
    check(xr, o, S, "erase_then_decay", TOL[dtype], "grouped %s d%d %s" % (kind, D, dtype))


def test_decode_grouped_heads(dev):
    import gated_delta_rule_71_amd as gdr
    from gpu_util import to_dev
    wl = case("gdn2", B=3, H=4, T=5, D=128, s0=0.02)
    xq, xr = grouped(synth.make_prefill(wl), 4)
    g = to_dev(xq, dev)
    S = g["S0"].clone()
    outs = []
    for t in range(wl.T):
        sl = lambda a: None if a is None else a[:, t:t + 1].contiguous()
        outs.append(gdr.decode_step(sl(g["q"]), sl(g["k"]), sl(g["v"]), sl(g["log_alpha"]),
                                    sl(g["b"]), sl(g["w"]), S))
    torch.cuda.synchronize()
    o = torch.cat(outs, dim=1)
    check(xr, o, S, "erase_then_decay", TOL["bf16"], "grouped decode")


# ------------------------------------------------------------------ d_k = 256


@pytest.mark.parametrize("kind,DV", [("gdn", 256), ("gdn", 64), ("la", 128), ("mamba2", 256),
                                     ("deltanet", 64)])
def test_prefill_dk256(dev, kind, DV):
    """d_k = 256 (the all-modes kernel with unpadded LDS rows): scalar, no or channel-free gates."""
    wl = case(kind, B=1, H=2, T=133, D=256, DV=DV, seed=101)
    say("prefill dk256", kind, DV)
    x = synth.make_prefill(wl)
    o, S = run_gpu_prefill(x, dev)
    torch.cuda.synchronize()
    check(x, o, S, "erase_then_decay", TOL["bf16"], "dk256 %s dv=%d" % (kind, DV))


def test_prefill_dk256_channel_decay_first(dev):
    """d_k = 256 with a per-channel decay applied before the erase (KDA gates)."""
    wl = case("kda", B=1, H=2, T=100, D=256, DV=64, seed=102)
    say("prefill dk256 kda decay first")
    x = synth.make_prefill(wl)
    o, S = run_gpu_prefill(x, dev, order="decay_then_erase")
    torch.cuda.synchronize()
    check(x, o, S, "decay_then_erase", TOL["bf16"], "dk256 kda decay first")


@pytest.mark.parametrize("kind,dtype", [("gdn2", "bf16"), ("gdn", "fp32")])
def test_decode_dk256(dev, kind, dtype):
    """One decode step at d_k = d_v = 256 against the oracle's single token from the same state."""
    import gated_delta_rule_71_amd as gdr
    from gpu_util import to_dev
    wl = case(kind, B=3, H=2, T=1, D=256, DV=256, dtype=dtype, s0=0.02, seed=103)
    say("decode dk256", kind, dtype)
    x = synth.make_prefill(wl)
    g = to_dev(x, dev)
    S = g["S0"].clone()
    o = gdr.decode_step(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], S)
    torch.cuda.synchronize()
    check(x, o, S, "erase_then_decay", TOL[dtype], "decode dk256 %s %s" % (kind, dtype))
