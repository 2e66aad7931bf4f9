"""State decomposition and causal interventions on the recurrence.

"How Linear Attention Remembers", Analytical Framework: with S_t = T_t(S_{t-1}) + W_t (T_t linear
in the state, W_t the write of token t), the state is a sum of per-position contributions

    S_t = sum_{i <= t} C_i^(t),   C_i^(t) = (T_t o ... o T_{i+1})(W_i),   C_i^(i) = W_i,

and its Causal Intervention Framework blocks or replaces the write at a fact position and swaps
the state before a query.  For the gated delta rule T_t(S) = Diag(alpha_t)(I - k_t^T c_t) S
(erase then decay; the other order swaps the factors) and W_t = k_t^T (w_t . v_t), so:

* C_i^(t) is the final state of the recurrence over tokens 0..t from a zero state with every
  write gate w_j set to zero except at j = i (the transitions are untouched);
* blocking the write at x is the same call with w_x = 0, and S_t(blocked) = S_t - C_x^(t);
* replacing it by a donor's write is, by linearity, the blocked run plus the donor's write
  carried through the recipient's transitions;
* a pre-query state swap continues the recipient's tokens from the donor's state.

Each function runs the recurrence through ``chunk_fwd`` (the HIP library); this module only
builds masked gate tensors.  Inputs are device tensors laid out as for ``chunk_fwd``.
"""
from . import chunk_fwd


def _torch():
    import torch
    return torch


def _write_gate(w, v, B, T, H):
    """The write gate as an explicit tensor (w = 1 when absent): [B, T, H] or [B, T, H, dv]."""
    torch = _torch()
    if w is not None:
        return w
    return torch.ones((B, T, H), dtype=v.dtype, device=v.device)


def _token_mask(w, keep, batch_rows=None):
    """w with every token outside `keep` (a bool [T] or [rows, T] tensor) zeroed."""
    m = keep.to(w.dtype)
    if m.dim() == 1:
        m = m.view(1, -1)
    while m.dim() < w.dim():
        m = m.unsqueeze(-1)
    return w * m


def contributions(q, k, v, log_alpha=None, b=None, w=None, positions=(0,), t=None,
                  order="erase_then_decay"):
    """C_i^(t) for every i in `positions` (0-based, i <= t; t defaults to the last token).

    Returns float32 [len(positions), B, H, dk, dv]: the contribution of each position's write to
    the state after token t.  One ``chunk_fwd`` call over len(positions) * B sequences of t + 1
    tokens, each keeping a single write."""
    torch = _torch()
    B, T, _, DK = q.shape
    H, DV = v.shape[2], v.shape[-1]
    t = T - 1 if t is None else int(t)
    pos = [int(i) for i in positions]
    if not 0 <= t < T or any(not 0 <= i <= t for i in pos):
        raise ValueError("positions must satisfy 0 <= i <= t < T")
    P, L = len(pos), t + 1

    def rep(x):
        if x is None:
            return None
        x = x[:, :L]
        return x.unsqueeze(0).expand(P, *x.shape).reshape(P * B, *x.shape[1:]).contiguous()

    wf = _write_gate(w, v, B, T, H)
    ww = rep(wf)
    keep = torch.zeros((P, L), dtype=torch.bool, device=v.device)
    keep[torch.arange(P, device=v.device), torch.tensor(pos, device=v.device)] = True
    keep = keep.unsqueeze(1).expand(P, B, L).reshape(P * B, L)
    ww = _token_mask(ww, keep)
    _, S = chunk_fwd(rep(q), rep(k), rep(v), rep(log_alpha), rep(b), ww, None, order=order)
    return S.view(P, B, H, DK, DV)


def block_write(q, k, v, log_alpha=None, b=None, w=None, S0=None, position=0, heads=None,
                order="erase_then_decay"):
    """The recurrence with the write at `position` removed (for the listed heads, or all).
    Returns (o, S_T) like ``chunk_fwd``."""
    torch = _torch()
    B, T, H = v.shape[:3]
    wf = _write_gate(w, v, B, T, H).clone()
    hs = slice(None) if heads is None else torch.as_tensor(heads, device=v.device)
    if wf.dim() == 3:
        wf[:, position, hs] = 0
    else:
        wf[:, position, hs, :] = 0
    return chunk_fwd(q, k, v, log_alpha, b, wf, S0, order=order)


def replace_write(q, k, v, log_alpha=None, b=None, w=None, S0=None, position=0, donor=None,
                  order="erase_then_decay"):
    """The recurrence with the write at `position` replaced by a donor's write there.

    `donor` is a dict with the donor's "k", "v" and (optionally) "w" tensors of the same shapes;
    only their values at `position` are used.  The erase and decay at `position` stay the
    recipient's.  Returns (o, S_T): the blocked run plus the donor write carried through the
    recipient's transitions (one ``chunk_fwd`` call over a batch of two).  The two runs' outputs
    are added in fp32 and o is rounded to the I/O dtype once more, so a bf16 o carries one rounding
    beyond that of a single run (at most half a bf16 unit in the last place); S_T is the fp32 sum
    of the two fp32 states."""
    torch = _torch()
    if donor is None:
        raise ValueError("replace_write needs the donor's tensors")
    B, T, H = v.shape[:3]
    wf = _write_gate(w, v, B, T, H)
    dw = _write_gate(donor.get("w"), donor["v"], B, T, H)
    if dw.dim() != wf.dim():
        raise ValueError("donor and recipient write gates must have the same kind")
    keep = torch.zeros(T, dtype=torch.bool, device=v.device)
    keep[position] = True
    # run 1: the recipient with the write blocked; run 2: only the donor's write, from zero
    w_blocked = _token_mask(wf, ~keep)
    k2, v2 = k.clone(), v.clone()
    k2[:, position] = donor["k"][:, position]
    v2[:, position] = donor["v"][:, position]
    w_donor = _token_mask(dw, keep)
    cat = lambda a, c: None if a is None else torch.cat([a, a if c is None else c], 0)
    S0s = None if S0 is None else torch.cat([S0, torch.zeros_like(S0)], 0)
    o, S = chunk_fwd(cat(q, None), torch.cat([k, k2], 0), torch.cat([v, v2], 0),
                     cat(log_alpha, None), cat(b, None), torch.cat([w_blocked, w_donor], 0), S0s,
                     order=order)
    return (o[:B].float() + o[B:].float()).to(o.dtype), S[:B] + S[B:]


def swap_state(q, k, v, log_alpha=None, b=None, w=None, S0=None, position=0, donor=None,
               order="erase_then_decay"):
    """Run the recipient's tokens 0..position, then swap in the donor's state after `position`
    (computed from the donor's tokens 0..position, same S0) and continue the recipient's tokens.

    `donor` is a dict with "q", "k", "v" and the donor's gates ("log_alpha", "b", "w") as used by
    ``chunk_fwd``.  Returns (o of tokens position+1.., S_T, recipient state before the swap,
    donor state swapped in)."""
    torch = _torch()
    if donor is None:
        raise ValueError("swap_state needs the donor's tensors")
    p = int(position) + 1
    head = lambda x: None if x is None else x[:, :p].contiguous()
    tail = lambda x: None if x is None else x[:, p:].contiguous()
    _, S_rec = chunk_fwd(head(q), head(k), head(v), head(log_alpha), head(b), head(w), S0, order=order)
    _, S_don = chunk_fwd(head(donor["q"]), head(donor["k"]), head(donor["v"]),
                         head(donor.get("log_alpha")), head(donor.get("b")), head(donor.get("w")),
                         S0, order=order)
    o, S_T = chunk_fwd(tail(q), tail(k), tail(v), tail(log_alpha), tail(b), tail(w),
                       S_don.contiguous(), order=order)
    return o, S_T, S_rec, S_don
