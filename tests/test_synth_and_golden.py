"""Input generator determinism and the oracle's regression fixture."""
import os

import numpy as np
import torch

import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def test_same_seed_same_bytes():
    wl = synth.WORKLOADS["gdn"].with_(B=1, H=2, T=128)
    a = synth.make_prefill(wl)
    b = synth.make_prefill(wl)
    for name in ("q", "k", "v", "log_alpha", "b"):
        assert a[name].dtype == torch.bfloat16
        assert torch.equal(a[name].view(torch.int16), b[name].view(torch.int16)), name
    c = synth.make_prefill(wl, seed=wl.seed + 1)
    assert not torch.equal(a["q"], c["q"])


def test_workload_shapes_and_ranges():
    wl = synth.WORKLOADS["gdn2"].with_(T=64)
    x = synth.make_prefill(wl)
    B, T, H, D = wl.B, wl.T, wl.H, wl.DK
    assert x["q"].shape == (B, T, H, D) and x["log_alpha"].shape == (B, T, H, D)
    assert x["b"].shape == (B, T, H, D) and x["w"].shape == (B, T, H, wl.DV)
    assert x["S0"].shape == (B, H, D, wl.DV) and x["S0"].dtype == torch.float32
    la = x["log_alpha"].float()
    assert (la < 0).all()
    assert ((x["b"].float() > 0) & (x["b"].float() < 1)).all()
    n = x["q"].float().pow(2).sum(-1).sqrt()
    assert torch.allclose(n, torch.ones_like(n), atol=1e-2)
    assert abs(x["S0"].std().item() - 0.02) < 2e-3
    g = synth.make_prefill(synth.WORKLOADS["gdn"].with_(T=64))
    assert g["log_alpha"].shape == (4, 64, 16) and g["w"] is g["b"]


def test_oracle_reproduces_golden_fixture():
    import importlib.util
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(HERE, "golden",
                                                                              "make_golden.py"))
    mg = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mg)
    rows = np.loadtxt(os.path.join(HERE, "golden", "tiny_oracle.txt"))
    o, S = mg.compute()
    np.testing.assert_allclose(np.vstack([o, S]), rows, rtol=1e-13, atol=1e-15)
