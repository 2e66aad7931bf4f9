"""The allocation-free prefill (gdr_chunk_fwd_noalloc) against gdr_chunk_fwd, through the C ABI.

Two calls in a row, the second with a smaller problem, each compared bit for bit with the ordinary
entry point given a caller workspace (the same kernels run on the same inputs), and against the
fp64 oracle at the bf16 tolerance (max |o - o_ref| <= 2e-2, per-state relative Frobenius error of
S_T <= 1e-2)."""
import sys

import numpy as np
import pytest

import synth
from gpu_util import TOL, errors, run_oracle, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_71_amd as gdr
    gdr._native.lib()
    return torch.device("cuda:0")


def problem_of(wl, x):
    import gated_delta_rule_71_amd as gdr
    N = gdr._native
    kind = lambda t: N.GATE_NONE if t is None else (N.GATE_SCALAR if t.dim() == 3 else N.GATE_CHANNEL)
    return gdr.make_problem(wl.B, wl.H, wl.T, wl.DK, wl.DV, N.GDR_BF16, kind(x["log_alpha"]),
                            kind(x["b"]), kind(x["w"]), N.ERASE_THEN_DECAY)


def run_both(wl, dev):
    import gated_delta_rule_71_amd as gdr
    N = gdr._native
    x = synth.make_prefill(wl)
    g = to_dev(x, dev)
    prob = problem_of(wl, x)
    need = N.workspace_bytes(prob)
    assert 0 < need <= N.NOALLOC_SCRATCH_BYTES, need
    ptr = lambda t: 0 if t is None else t.data_ptr()
    stream = torch.cuda.current_stream(dev).cuda_stream
    outs = []
    for noalloc in (False, True):
        o = torch.full((wl.B, wl.T, wl.H, wl.DV), float("nan"), dtype=torch.bfloat16, device=dev)
        S = torch.full((wl.B, wl.H, wl.DK, wl.DV), float("nan"), dtype=torch.float32, device=dev)
        args = [ptr(g[n]) for n in ("q", "k", "v", "log_alpha", "b", "w", "S0")] + [ptr(o), ptr(S)]
        if noalloc:
            rc = N.chunk_fwd_noalloc_raw(prob, *args, stream)
        else:
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
            rc = N.chunk_fwd_raw(prob, *args, ptr(ws), need, stream)
        assert rc == N.GDR_OK, N.status_string(rc)
        torch.cuda.synchronize()
        outs.append((o, S))
    (o1, S1), (o2, S2) = outs
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    o_ref, S_ref = run_oracle(x)
    eo, es = errors(o2, S2, o_ref, S_ref)
    say("noalloc %s B=%d H=%d T=%d: max|do|=%.3e rel|dS|=%.3e" % (wl.name, wl.B, wl.H, wl.T, eo, es))
    assert eo <= TOL["bf16"][0] and es <= TOL["bf16"][1]


@pytest.mark.parametrize("name", ["gdn2", "gdn", "kda"])
def test_noalloc_matches_the_workspace_entry_point(dev, name):
    wl = synth.WORKLOADS[name].with_(B=2, H=4, T=700)
    run_both(wl, dev)
    run_both(wl.with_(B=1, H=2, T=130), dev)  # second call, smaller input
