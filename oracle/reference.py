"""NumPy fp64 twins of the recurrence, used to pin the C oracle (test infrastructure only).

Every function works on arrays laid out ``[B, T, H, D]`` (gates ``[B, T, H]`` for
a scalar per token and head, ``[B, T, H, D]`` per channel, or ``None``) and
returns float64.  Each one is written from the pages independently of
``gdr_oracle.c``:

* ``recurrence_operator`` -- the unified equation of "Recurrent Memory: Write,
  Erase, Decay, Read" section 05, applied literally as a dk x dk transition
  matrix Diag(alpha_t)(I - k_t^T c_t) times S plus the rank-one write, with
  the Gated DeltaNet-2 gates (c_t = b_t . k_t, written value w_t . v_t).
* ``linear_attention_masked`` / ``gla_masked`` -- the "structured masked
  matrix" view of State Space Duality ("The Eraser Trilogy", The Rosetta
  Stone): with the erase off, o_t = sum_{i<=t} (q_t . (Gamma_t/Gamma_i) . k_i) x_i.
* ``deltanet_three_line`` -- the three-line delta rule of section 03 (read,
  delta, write back), with beta as a scalar.
* ``chunkwise`` -- the chunk (WY/UT) form: gate prefix sums inside each chunk,
  a unit-lower-triangular solve for the erase reads, and a state hand-off
  between chunks.  It is derived by unrolling the recurrence over a chunk
  (section 03: the erase is linear, so it reassociates into a chunkwise form;
  section 04: survival is exp of a prefix sum of log alpha).
"""
import numpy as np


def _gate(g, B, T, H, D, default):
    """Expand a gate to [B, T, H, D] float64 (scalar gates broadcast over channels)."""
    if g is None:
        return np.full((B, T, H, D), default, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    if g.ndim == 3:
        return np.broadcast_to(g[..., None], (B, T, H, D)).copy()
    return g.copy()


def _unpack(q, k, v, log_alpha, b, w):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    la = _gate(log_alpha, B, T, H, DK, 0.0)
    bb = _gate(b, B, T, H, DK, 0.0)
    ww = _gate(w, B, T, H, DV, 1.0)
    return q, k, v, la, bb, ww, (B, T, H, DK, DV)


def _s0(S0, B, H, DK, DV):
    if S0 is None:
        return np.zeros((B, H, DK, DV), dtype=np.float64)
    return np.array(S0, dtype=np.float64, copy=True)


def recurrence_operator(q, k, v, log_alpha=None, b=None, w=None, S0=None, order=0):
    """S_t = A_t S_{t-1} + k_t^T x_t with A_t = Diag(alpha_t)(I - k_t^T c_t) (order 0)
    or (I - k_t^T c_t) Diag(alpha_t) (order 1); o_t = q_t S_t."""
    q, k, v, la, bb, ww, (B, T, H, DK, DV) = _unpack(q, k, v, log_alpha, b, w)
    S = _s0(S0, B, H, DK, DV)
    o = np.zeros((B, T, H, DV))
    eye = np.eye(DK)
    for bi in range(B):
        for hi in range(H):
            St = S[bi, hi]
            for t in range(T):
                kt, ct = k[bi, t, hi], bb[bi, t, hi] * k[bi, t, hi]
                Dm = np.diag(np.exp(la[bi, t, hi]))
                E = eye - np.outer(kt, ct)
                A = Dm @ E if order == 0 else E @ Dm
                St = A @ St + np.outer(kt, ww[bi, t, hi] * v[bi, t, hi])
                o[bi, t, hi] = q[bi, t, hi] @ St
            S[bi, hi] = St
    return o, S


def contribution(q, k, v, log_alpha=None, b=None, w=None, i=0, t=None, order=0, write=None):
    """C_i^(t) = (T_t o ... o T_{i+1})(W_i), C_i^(i) = W_i ("How Linear Attention Remembers",
    Analytical Framework), with T_j(S) = A_j S as in recurrence_operator and the rank-one write
    W_i = k_i^T (w_i . v_i), or W_i = k^T x for write = (k, x) given per (batch, head) as
    arrays [B, H, DK] and [B, H, DV].  Returns [B, H, DK, DV] float64."""
    q, k, v, la, bb, ww, (B, T, H, DK, DV) = _unpack(q, k, v, log_alpha, b, w)
    t = T - 1 if t is None else t
    C = np.zeros((B, H, DK, DV))
    eye = np.eye(DK)
    for bi in range(B):
        for hi in range(H):
            if write is None:
                Ci = np.outer(k[bi, i, hi], ww[bi, i, hi] * v[bi, i, hi])
            else:
                Ci = np.outer(np.asarray(write[0], dtype=np.float64)[bi, hi],
                              np.asarray(write[1], dtype=np.float64)[bi, hi])
            for j in range(i + 1, t + 1):
                kt, ct = k[bi, j, hi], bb[bi, j, hi] * k[bi, j, hi]
                Dm = np.diag(np.exp(la[bi, j, hi]))
                E = eye - np.outer(kt, ct)
                Ci = (Dm @ E if order == 0 else E @ Dm) @ Ci
            C[bi, hi] = Ci
    return C


def linear_attention_masked(q, k, x):
    """Erase off, alpha = 1: O = tril(Q K^T) X per (batch, head)."""
    q, k, x = (np.asarray(a, dtype=np.float64) for a in (q, k, x))
    B, T, H, _ = q.shape
    o = np.zeros(x.shape)
    mask = np.tril(np.ones((T, T)))
    for bi in range(B):
        for hi in range(H):
            A = (q[bi, :, hi] @ k[bi, :, hi].T) * mask
            o[bi, :, hi] = A @ x[bi, :, hi]
    return o


def gla_masked(q, k, x, log_alpha):
    """Erase off, decay on (scalar or per channel), S0 = 0:
    o_t = sum_{i<=t} sum_d q_td k_id exp(G_td - G_id) x_i with G the prefix sum of log alpha."""
    q, k, x = (np.asarray(a, dtype=np.float64) for a in (q, k, x))
    B, T, H, DK = q.shape
    la = _gate(log_alpha, B, T, H, DK, 0.0)
    G = np.cumsum(la, axis=1)
    o = np.zeros(x.shape)
    for bi in range(B):
        for hi in range(H):
            Gh = G[bi, :, hi]
            for t in range(T):
                dec = np.exp(Gh[t][None, :] - Gh[: t + 1])  # [i, d], exponent <= 0
                wts = (dec * k[bi, : t + 1, hi] * q[bi, t, hi][None, :]).sum(axis=1)
                o[bi, t, hi] = wts @ x[bi, : t + 1, hi]
    return o


def deltanet_three_line(q, k, v, beta, S0=None):
    """Section 03's delta rule with alpha = 1 and scalar beta:
    v_old = k_t S; u_t = beta_t (v_t - v_old); S <- S + k_t^T u_t; o_t = q_t S."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    beta = np.asarray(beta, dtype=np.float64)
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    S = _s0(S0, B, H, DK, DV)
    o = np.zeros((B, T, H, DV))
    for bi in range(B):
        for hi in range(H):
            St = S[bi, hi]
            for t in range(T):
                v_old = k[bi, t, hi] @ St
                u = beta[bi, t, hi] * (v[bi, t, hi] - v_old)
                St = St + np.outer(k[bi, t, hi], u)
                o[bi, t, hi] = q[bi, t, hi] @ St
            S[bi, hi] = St
    return o, S


def chunkwise(q, k, v, log_alpha=None, b=None, w=None, S0=None, order=0, chunk=64):
    """Chunk form of the recurrence, fp64.  Inside a chunk of n tokens with entering state S
    and local prefix sums G_t (G_0 = 0):

    erase then decay (order 0):
        Chat_t = c_t e^{G_{t-1}},  Khat_i = k_i e^{-G_i},  Phat_i = k_i e^{-G_{i-1}},  Qhat_t = q_t e^{G_t}
        (I + strict_tril(Chat Phat^T)) R = Chat S + strict_tril(Chat Khat^T) X      (R_t = c_t S_{t-1})
        O   = Qhat S + tril(Qhat Khat^T) X - tril(Qhat Phat^T) R
        S'  = e^{G_n} . S + Kbar^T X - Pbar^T R,  Kbar_i = k_i e^{G_n - G_i},  Pbar_i = k_i e^{G_n - G_{i-1}}
    decay then erase (order 1):
        Chat_t = c_t e^{G_t};  (I + strict_tril(Chat Khat^T)) U = X - Chat S
        O = Qhat S + tril(Qhat Khat^T) U;  S' = e^{G_n} . S + Kbar^T U
    """
    q, k, v, la, bb, ww, (B, T, H, DK, DV) = _unpack(q, k, v, log_alpha, b, w)
    S = _s0(S0, B, H, DK, DV)
    o = np.zeros((B, T, H, DV))
    c_all = bb * k
    x_all = ww * v
    for bi in range(B):
        for hi in range(H):
            St = S[bi, hi]
            for s in range(0, T, chunk):
                e = min(s + chunk, T)
                n = e - s
                qc, kc = q[bi, s:e, hi], k[bi, s:e, hi]
                cc, xc = c_all[bi, s:e, hi], x_all[bi, s:e, hi]
                G = np.cumsum(la[bi, s:e, hi], axis=0)
                Gp = np.vstack([np.zeros((1, DK)), G[:-1]])
                Gn = G[-1]
                Kh = kc * np.exp(-G)
                Qh = qc * np.exp(G)
                Kb = kc * np.exp(Gn[None, :] - G)
                I = np.eye(n)
                if order == 0:
                    Ch = cc * np.exp(Gp)
                    Ph = kc * np.exp(-Gp)
                    Pb = kc * np.exp(Gn[None, :] - Gp)
                    LP = np.tril(Ch @ Ph.T, -1)
                    LK = np.tril(Ch @ Kh.T, -1)
                    R = np.linalg.solve(I + LP, Ch @ St + LK @ xc)
                    o[bi, s:e, hi] = Qh @ St + np.tril(Qh @ Kh.T) @ xc - np.tril(Qh @ Ph.T) @ R
                    St = np.exp(Gn)[:, None] * St + Kb.T @ xc - Pb.T @ R
                else:
                    Ch = cc * np.exp(G)
                    L = np.tril(Ch @ Kh.T, -1)
                    U = np.linalg.solve(I + L, xc - Ch @ St)
                    o[bi, s:e, hi] = Qh @ St + np.tril(Qh @ Kh.T) @ U
                    St = np.exp(Gn)[:, None] * St + Kb.T @ U
            S[bi, hi] = St
    return o, S
