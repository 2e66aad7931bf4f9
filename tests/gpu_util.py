"""Helpers shared by the GPU tests: running the HIP path and the oracle on the same inputs."""
import numpy as np

import oracle
import synth

# Tolerances: bf16 inputs with an fp32 state; all-fp32 mode.
TOL = {"bf16": (2e-2, 1e-2), "fp32": (1e-4, 1e-4)}  # (max |do|, max per-state rel Frobenius dS)


def to_dev(x, dev):
    return {n: (None if t is None else t.to(dev)) for n, t in x.items()}


def run_gpu_prefill(x, dev, order="erase_then_decay"):
    import gated_delta_rule_71_amd as gdr
    g = to_dev(x, dev)
    o, S_T = gdr.chunk_fwd(g["q"], g["k"], g["v"], g["log_alpha"], g["b"], g["w"], g["S0"],
                           order=order)
    return o, S_T


def run_oracle(x, order=0):
    return oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], x["S0"],
                          order=order)


def errors(o_gpu, S_gpu, o_ref, S_ref):
    o = o_gpu.float().cpu().numpy().astype(np.float64)
    err_o = float(np.abs(o - o_ref).max()) if o.size else 0.0
    if S_gpu is None:
        return err_o, 0.0
    S = S_gpu.cpu().numpy().astype(np.float64)
    n = S.shape[0] * S.shape[1]
    d = np.linalg.norm((S - S_ref).reshape(n, -1), axis=1)
    r = np.linalg.norm(S_ref.reshape(n, -1), axis=1)
    rel = float((d / np.maximum(r, 1e-30)).max()) if n else 0.0
    return err_o, rel


def subset_heads(x, b_idx, h_idx):
    """Inputs of selected (batch, head) pairs as a [len, T, 1, D] problem for the oracle."""
    out = {}
    for n, t in x.items():
        if t is None:
            out[n] = None
        elif n == "S0":
            out[n] = t[b_idx, h_idx][:, None]
        else:
            out[n] = t[b_idx, :, h_idx].unsqueeze(2) if t.dim() == 4 else t[b_idx, :, h_idx].unsqueeze(2)
    return out


def workload(name, **kw):
    return synth.WORKLOADS[name].with_(**kw)
