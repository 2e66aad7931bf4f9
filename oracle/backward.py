"""Reverse-mode gradient of the gated delta-rule recurrence in fp64 (test infrastructure only).

The forward is the unified recurrence of "Recurrent Memory: Write, Erase, Decay, Read" (section
05) with the Gated DeltaNet-2 gates: per token t, with c_t = b_t . k_t and x_t = w_t . v_t,

    erase then decay (order 0):  r_t = c_t S_{t-1},  P_t = S_{t-1} - k_t^T r_t,
                                 S_t = Diag(alpha_t) P_t + k_t^T x_t
    decay then erase (order 1):  P_t = Diag(alpha_t) S_{t-1},  r_t = c_t P_t,
                                 S_t = P_t - k_t^T r_t + k_t^T x_t

and o_t = q_t S_t (alpha_t = exp(log alpha_t)).  Given the gradients do of every output and dS_T
of the final state, ``backward`` walks the tokens in reverse holding G = dL/dS_t and applies the
chain rule to each line above, one token at a time; the forward states are recomputed and kept.
Nothing here is blocked, chunked or reordered: it is the adjoint of the token loop, checked
against central finite differences of ``reference.recurrence_operator`` (a separate forward in
operator form) on tiny inputs.
"""
import numpy as np

from .reference import _gate


def _reduce_like(g_full, g_in):
    """Gradient of a gate expanded per channel, summed back to the gate's own shape."""
    if g_in is None:
        return None
    if np.ndim(g_in) == 3:
        return g_full.sum(axis=-1)
    return g_full


def backward(q, k, v, log_alpha=None, b=None, w=None, S0=None, do=None, dS_T=None, order=0):
    """Gradients of L = <do, o> + <dS_T, S_T> with respect to every input.

    Shapes as for the forward: q, k [B, T, H, DK]; v [B, T, H, DV]; each gate [B, T, H]
    (scalar per token and head), [B, T, H, D] (per channel) or None (log alpha = 0, b = 0,
    w = 1); S0 [B, H, DK, DV] or None; do [B, T, H, DV]; dS_T [B, H, DK, DV] or None.
    Returns a dict of float64 arrays shaped like the inputs: dq, dk, dv, dlog_alpha, db, dw
    (None where the gate is None) and dS0."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    N = B * H
    la = _gate(log_alpha, B, T, H, DK, 0.0)
    bb = _gate(b, B, T, H, DK, 0.0)
    ww = _gate(w, B, T, H, DV, 1.0)
    # per (batch, head) chains: [N, T, D]
    tr = lambda x: np.ascontiguousarray(np.transpose(x, (0, 2, 1, 3)).reshape(N, T, x.shape[-1]))
    q_, k_, v_, la_, b_, w_ = tr(q), tr(k), tr(v), tr(la), tr(bb), tr(ww)
    do_ = tr(np.asarray(do, dtype=np.float64)) if do is not None else np.zeros((N, T, DV))
    al = np.exp(la_)
    c_ = b_ * k_
    x_ = w_ * v_
    S = np.zeros((N, DK, DV)) if S0 is None else np.array(S0, dtype=np.float64).reshape(N, DK, DV)

    # forward, keeping S_{t-1} for every token
    Sprev = np.empty((T, N, DK, DV))
    for t in range(T):
        Sprev[t] = S
        kt, ct, at, xt = k_[:, t], c_[:, t], al[:, t], x_[:, t]
        if order == 0:
            r = np.einsum("ni,nij->nj", ct, S)
            P = S - kt[:, :, None] * r[:, None, :]
            S = at[:, :, None] * P + kt[:, :, None] * xt[:, None, :]
        else:
            P = at[:, :, None] * S
            r = np.einsum("ni,nij->nj", ct, P)
            S = P - kt[:, :, None] * r[:, None, :] + kt[:, :, None] * xt[:, None, :]

    dq_, dk_, dx_, dla_, dc_ = (np.zeros_like(q_), np.zeros_like(k_), np.zeros_like(x_),
                                np.zeros_like(la_), np.zeros_like(c_))
    G = np.zeros((N, DK, DV)) if dS_T is None else np.array(dS_T, dtype=np.float64).reshape(N, DK, DV)
    St = S  # S_t for the token being undone
    for t in range(T - 1, -1, -1):
        Sp = Sprev[t]
        qt, kt, ct, at, xt, dot = q_[:, t], k_[:, t], c_[:, t], al[:, t], x_[:, t], do_[:, t]
        # o_t = q_t S_t
        dq_[:, t] = np.einsum("nij,nj->ni", St, dot)
        G = G + qt[:, :, None] * dot[:, None, :]
        # the write k_t^T x_t
        dx_[:, t] = np.einsum("ni,nij->nj", kt, G)
        dkt = np.einsum("nij,nj->ni", G, xt)
        if order == 0:
            r = np.einsum("ni,nij->nj", ct, Sp)
            P = Sp - kt[:, :, None] * r[:, None, :]
            dal = np.einsum("nij,nij->ni", G, P)         # S_t = Diag(alpha) P + ...
            dP = at[:, :, None] * G
            dr = -np.einsum("ni,nij->nj", kt, dP)        # P = S_{t-1} - k^T r
            dkt -= np.einsum("nij,nj->ni", dP, r)
            dc_[:, t] = np.einsum("nij,nj->ni", Sp, dr)   # r = c S_{t-1}
            G = dP + ct[:, :, None] * dr[:, None, :]
        else:
            P = at[:, :, None] * Sp
            r = np.einsum("ni,nij->nj", ct, P)
            dr = -np.einsum("ni,nij->nj", kt, G)         # S_t = P - k^T r + ...
            dkt -= np.einsum("nij,nj->ni", G, r)
            dP = G + ct[:, :, None] * dr[:, None, :]     # r = c P
            dc_[:, t] = np.einsum("nij,nj->ni", P, dr)
            dal = np.einsum("nij,nij->ni", dP, Sp)       # P = Diag(alpha) S_{t-1}
            G = at[:, :, None] * dP
        dla_[:, t] = dal * at                            # alpha = exp(log alpha)
        dk_[:, t] = dkt
        St = Sp

    # c = b . k and x = w . v
    dk_ += dc_ * b_
    db_ = dc_ * k_
    dv_ = dx_ * w_
    dw_ = dx_ * v_
    un = lambda x: np.transpose(x.reshape(B, H, T, x.shape[-1]), (0, 2, 1, 3))
    return {
        "dq": un(dq_), "dk": un(dk_), "dv": un(dv_),
        "dlog_alpha": _reduce_like(un(dla_), log_alpha),
        "db": _reduce_like(un(db_), b),
        "dw": _reduce_like(un(dw_), w),
        "dS0": G.reshape(B, H, DK, DV),
    }
