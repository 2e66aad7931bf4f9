"""Seeded synthetic inputs for the gated delta-rule workloads.

This module only draws random numbers and applies the input transforms that
define the workloads (row L2-normalisation of q and k, sigmoid for the erase
and write gates, -softplus for the log-decay, rounding to the I/O dtype).  It
holds none of the recurrence's arithmetic, so both the CPU oracle's tests and
the GPU path's tests and benchmark can draw their inputs from it.

Workloads (shapes follow the recurrent heads of the "How Linear Attention
Remembers" appendix table: H heads with d_k = d_v = 128):

  tiny    B=1  H=1  T=64     d=16   fp32, scalar decay and beta, mu=0
  gdn     B=4  H=16 T=4096   d=128  bf16, scalar decay and beta        (Gated DeltaNet)
  kda     B=2  H=32 T=8192   d=128  bf16, per-channel decay, scalar beta (KDA)
  gdn2    B=1  H=16 T=32768  d=128  bf16, per-channel decay, b and w,   (Gated DeltaNet-2)
                                     S0 ~ N(0, 0.02^2)
  decode  B=256 H=32 d=128, one token per step, Gated DeltaNet-2 gates,
          S ~ N(0, 0.02^2), 1000 steps
  mamba2  B=4  H=16 T=4096   d=128  bf16, scalar decay, no erase, w = 1
  gla     B=4  H=16 T=4096   d=128  bf16, per-channel decay, no erase, w = 1
  gdn_gqa B=4  H=32 T=4096   d=128  bf16, as gdn with 16 shared q / k heads
  gdn_d256 B=4 H=8  T=4096   d=256  bf16, as gdn at d_k = d_v = 256

Distributions: q, k ~ N(0, 1) rows then L2-normalised; v ~ N(0, 1);
beta, b, w = sigmoid(N(0, 1)); log alpha = -softplus(N(mu, 1)) with mu = 0 for
``tiny`` and mu = -2 otherwise.  Host draws use NumPy's PCG64 with seed
``1000 + index``; values are drawn in float32 and rounded to the I/O dtype with
round-to-nearest-even.
"""
from dataclasses import dataclass, replace

import numpy as np

NONE, SCALAR, CHANNEL = "none", "scalar", "channel"


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    DK: int
    DV: int
    dtype: str          # "bf16" or "fp32": dtype of q, k, v, gates and o
    alpha: str          # none / scalar / channel
    b: str              # none / scalar / channel
    w: str              # none / scalar / channel
    shared_beta: bool   # b and w are the same scalar beta (Gated DeltaNet, KDA)
    mu: float           # mean of the pre-softplus decay logits
    s0_std: float       # 0 -> S0 = 0
    seed: int
    steps: int = 0      # decode workloads: consecutive steps
    HK: int = 0         # q / k heads (0: H); H a multiple of HK (grouped key / value heads)

    def with_(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 64, 16, 16, "fp32", SCALAR, SCALAR, SCALAR, True, 0.0, 0.0, 1000),
    "gdn": Workload("gdn", 4, 16, 4096, 128, 128, "bf16", SCALAR, SCALAR, SCALAR, True, -2.0, 0.0, 1001),
    "kda": Workload("kda", 2, 32, 8192, 128, 128, "bf16", CHANNEL, SCALAR, SCALAR, True, -2.0, 0.0, 1002),
    "gdn2": Workload("gdn2", 1, 16, 32768, 128, 128, "bf16", CHANNEL, CHANNEL, CHANNEL, False, -2.0,
                     0.02, 1003),
    "decode": Workload("decode", 256, 32, 1, 128, 128, "bf16", CHANNEL, CHANNEL, CHANNEL, False, -2.0,
                       0.02, 1004, steps=1000),
    # erase off (b = 0): linear attention with a scalar data-dependent decay (Mamba-2 style) at
    # the Gated DeltaNet shapes; w = 1
    "mamba2": Workload("mamba2", 4, 16, 4096, 128, 128, "bf16", SCALAR, NONE, NONE, False, -2.0, 0.0,
                       1005),
    # erase off with a per-channel decay (gated linear attention) at the Gated DeltaNet shapes; w = 1
    "gla": Workload("gla", 4, 16, 4096, 128, 128, "bf16", CHANNEL, NONE, NONE, False, -2.0, 0.0, 1007),
    # Gated DeltaNet gates at d_k = d_v = 256 (half the heads, the same state bytes per head-pair)
    "gdn_d256": Workload("gdn_d256", 4, 8, 4096, 256, 256, "bf16", SCALAR, SCALAR, SCALAR, True, -2.0, 0.0,
                         1008),
    # Gated DeltaNet gates with grouped heads: 32 value heads sharing 16 query / key heads
    "gdn_gqa": Workload("gdn_gqa", 4, 32, 4096, 128, 128, "bf16", SCALAR, SCALAR, SCALAR, True, -2.0,
                        0.0, 1006, HK=16),
}


def _torch_dtype(name):
    import torch
    return {"bf16": torch.bfloat16, "fp32": torch.float32}[name]


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _neg_softplus(x):
    # -softplus(x) = -(max(x, 0) + log1p(exp(-|x|))), stable for any x
    return -(np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x))))


def _l2rows(x):
    return x / np.sqrt((x.astype(np.float64) ** 2).sum(-1, keepdims=True)).astype(np.float32)


def make_prefill(wl, seed=None):
    """Host-side inputs for one prefill call.  Returns a dict of CPU torch tensors:
    q, k [B,T,HK or H,DK]; v [B,T,H,DV]; log_alpha, b, w ([B,T,H], [B,T,H,D] or None) in the
    workload's I/O dtype; S0 [B,H,DK,DV] float32 or None."""
    import torch
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    B, T, H, DK, DV = wl.B, wl.T, wl.H, wl.DK, wl.DV
    f32 = np.float32

    def normal(*shape):
        return rng.standard_normal(shape, dtype=f32)

    HQ = wl.HK or H
    q = _l2rows(normal(B, T, HQ, DK))
    k = _l2rows(normal(B, T, HQ, DK))
    v = normal(B, T, H, DV)
    gshape = {NONE: None, SCALAR: (B, T, H), CHANNEL: (B, T, H, DK)}
    la = None if wl.alpha == NONE else _neg_softplus(normal(*gshape[wl.alpha]) + f32(wl.mu)).astype(f32)
    if wl.shared_beta:
        beta = _sigmoid(normal(B, T, H)).astype(f32)
        b = beta if wl.b != NONE else None
        w = beta if wl.w != NONE else None
    else:
        b = None if wl.b == NONE else _sigmoid(normal(*gshape[wl.b])).astype(f32)
        wshape = {NONE: None, SCALAR: (B, T, H), CHANNEL: (B, T, H, DV)}[wl.w]
        w = None if wl.w == NONE else _sigmoid(normal(*wshape)).astype(f32)
    S0 = None
    if wl.s0_std > 0:
        S0 = (normal(B, H, DK, DV) * f32(wl.s0_std)).astype(f32)

    dt = _torch_dtype(wl.dtype)

    def to_t(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dt)

    out = dict(q=to_t(q), k=to_t(k), v=to_t(v), log_alpha=to_t(la), b=to_t(b), w=to_t(w),
               S0=None if S0 is None else torch.from_numpy(S0))
    if wl.shared_beta and b is not None and w is not None:
        out["w"] = out["b"]  # one beta buffer serves as both gates
    return out


def expand_heads(x, H):
    """q and k repeated per group so that every value head has its own copy (value head h reads
    q / k head h // (H // HK)); other entries unchanged."""
    out = dict(x)
    for n in ("q", "k"):
        G = H // x[n].shape[2]
        if G > 1:
            out[n] = x[n].repeat_interleave(G, dim=2)
    return out


def make_decode_state(wl, device, seed=None):
    """Decode state S [B,H,DK,DV] float32 ~ N(0, s0_std^2), drawn on `device` with torch's
    seeded generator (the state is 537 MB at the decode workload's size)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed if seed is None else seed)
    S = torch.randn((wl.B, wl.H, wl.DK, wl.DV), generator=g, device=device, dtype=torch.float32)
    return S.mul_(wl.s0_std)


def make_decode_steps(wl, n_steps, device, seed=None):
    """Per-step decode inputs drawn on `device` with torch's seeded generator:
    dict of tensors with a leading step axis, q,k [n,B,1,H,DK], v [n,B,1,H,DV],
    log_alpha/b [n,B,1,H,DK] (or [n,B,1,H] for scalar kinds), w [n,B,1,H,DV]."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((wl.seed if seed is None else seed) + 7919)
    B, H, DK, DV = wl.B, wl.H, wl.DK, wl.DV
    dt = _torch_dtype(wl.dtype)

    def normal(*shape):
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32)

    def l2(x):
        return x / x.double().pow(2).sum(-1, keepdim=True).sqrt().float()

    n = n_steps
    q = l2(normal(n, B, 1, H, DK)).to(dt)
    k = l2(normal(n, B, 1, H, DK)).to(dt)
    v = normal(n, B, 1, H, DV).to(dt)
    gs = {SCALAR: (n, B, 1, H), CHANNEL: (n, B, 1, H, DK)}
    la = None if wl.alpha == NONE else (-torch.nn.functional.softplus(normal(*gs[wl.alpha]) + wl.mu)).to(dt)
    if wl.shared_beta:
        beta = torch.sigmoid(normal(n, B, 1, H)).to(dt)
        b = beta if wl.b != NONE else None
        w = beta if wl.w != NONE else None
    else:
        b = None if wl.b == NONE else torch.sigmoid(normal(*gs[wl.b])).to(dt)
        ws = {SCALAR: (n, B, 1, H), CHANNEL: (n, B, 1, H, DV)}.get(wl.w)
        w = None if wl.w == NONE else torch.sigmoid(normal(*ws)).to(dt)
    return dict(q=q, k=k, v=v, log_alpha=la, b=b, w=w)
