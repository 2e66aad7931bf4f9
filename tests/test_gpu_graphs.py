"""The prefill and the decode step captured in a HIP graph (torch.cuda.CUDAGraph over the
binding, which passes the capturing stream to the C ABI) and replayed.

The library launches kernels only (no memset, copy or allocation inside a call), so a captured
call must give the eager call's bits on every replay.  Each replay is followed by eager work on
the same buffers (clearing them, an eager call) before the next, and every replay is compared
with the eager result."""
import sys

import pytest

import synth
from gpu_util import to_dev

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


PREFILL_CASES = {
    # name: (workload, overrides) -- one per kernel family
    "segment": ("gdn2", dict(B=1, H=4, T=300)),            # seg_kernel, chain and correction
    "two_kernel": ("gdn", dict(B=2, H=3, T=200, DK=64, DV=64)),  # chunk-local + per-state
    "fused": ("gdn", dict(B=2, H=2, T=150, DK=16, DV=32)),   # the all-modes kernel
    "recurrence": ("kda", dict(B=1, H=2, T=70, dtype="fp32")),  # the token recurrence (fp32, d = 128)
}


@pytest.mark.parametrize("case", list(PREFILL_CASES))
def test_prefill_graph_replays(dev, case):
    import gated_delta_rule_71_amd as gdr
    name, over = PREFILL_CASES[case]
    wl = synth.WORKLOADS[name].with_(**over)
    g = to_dev(synth.make_prefill(wl), dev)
    args = (g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], g["S0"])
    need = gdr.workspace_bytes(g["q"], g["v"], g["log_alpha"], g["b"], g["w"])
    ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    o_ref, S_ref = gdr.chunk_fwd(*args, workspace=ws)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):  # one call on the capture's stream before capturing
        gdr.chunk_fwd(*args, workspace=ws)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        o_g, S_g = gdr.chunk_fwd(*args, workspace=ws)
    for rep in range(3):
        o_g.zero_()
        S_g.zero_()
        graph.replay()
        torch.cuda.synchronize()
        say("prefill graph", case, "replay", rep)
        assert torch.equal(o_g, o_ref), (case, rep)
        assert torch.equal(S_g, S_ref), (case, rep)
        o_e, S_e = gdr.chunk_fwd(*args, workspace=ws)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(o_e, o_ref) and torch.equal(S_e, S_ref)


@pytest.mark.parametrize("io", ["bf16", "fp32"])
def test_decode_graph_replays(dev, io):
    """Three captured decode steps on one state buffer against three eager steps on a copy: the
    states and every step's read-out equal bit for bit."""
    import gated_delta_rule_71_amd as gdr
    dw = synth.WORKLOADS["decode"].with_(B=4, H=4, dtype=io)
    S0 = synth.make_decode_state(dw, dev)
    steps = synth.make_decode_steps(dw, 1, dev)
    t = {n: (None if v is None else v[0]) for n, v in steps.items()}
    args = (t["q"], t["k"], t["v"], t["log_alpha"], t["b"], t["w"])
    S_g = S0.clone()
    S_e = S0.clone()
    S_w = S0.clone()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        gdr.decode_step(*args, S=S_w)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        o_g = gdr.decode_step(*args, S=S_g)
    torch.cuda.synchronize()
    assert torch.equal(S_g, S0)  # capturing ran nothing
    for rep in range(3):
        graph.replay()
        o_e = gdr.decode_step(*args, S=S_e)
        torch.cuda.synchronize()
        say("decode graph", io, "replay", rep)
        assert torch.equal(o_g, o_e), (io, rep)
        assert torch.equal(S_g, S_e), (io, rep)
