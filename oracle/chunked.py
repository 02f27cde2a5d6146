"""Chunk-level quantities of the Gated DeltaNet forward, numpy fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Notation per value head and chunk of C tokens (rows r = 0..C-1):
  K, Q [C, d_k], V [C, d_v], g, beta [C]; state h [d_k, d_v].
  G_r   = sum_{s<=r} g_s                       (inclusive decay cumsum; G_last = G[C-1])
  Gam_ri = exp(G_r - G_i)                      (decay from token i to token r, i <= r)
  S_ri  = beta_r Gam_ri k_r.k_i   for i < r, else 0   (gated strict-lower beta*K*K^T)
  T     = (I + S)^-1                           (unit lower triangular, the "UT transform")
  W     = T diag(beta e^G) K,   U = T diag(beta) V,   K_g = diag(e^{G_last - G}) K
  A     = e^{G_last} I - K_g^T W,   B = K_g^T U           (h_end = A h + B)
  Delta = U - W h
  O     = diag(e^G) Q h + (Q K^T o Gam o [i <= r]) Delta

The pages name these objects without defining them: the inter-chunk step
h' = (exp(g_last) I - k_g^T w) h + k_g^T u = A h + B ("Shard the GatedDeltaNet
sequence under ici_context_parallelism", PR description; "GatedDeltaNet does
not support ici_context_parallelism", section "The recurrence is affine, so it
can be parallelized") and the triangular inverse A = (I+S)^-1 of the UT
transform ("Fuse the Gated Delta Net inter-chunk scan into a Pallas TPU
kernel", section "Changes", triangular-inversion item).  The definitions
above are the reading under which that step equals the per-token rule
S_t = exp(g_t)(I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T, o_t = S_t^T q_t,
which the CPU tests check to ~1e-15.
"""
from __future__ import annotations

import numpy as np


def decay_cumsum(g):
    """G_r = sum_{s<=r} g_s (inclusive), the log-decay from the chunk start."""
    return np.cumsum(np.asarray(g, np.float64))


def decay_matrix(G):
    """Gam_ri = exp(G_r - G_i) for i <= r, 0 above the diagonal.
    The exponent is masked before exp: above the diagonal it is positive and
    may overflow."""
    G = np.asarray(G, np.float64)
    C = G.shape[0]
    diff = G[:, None] - G[None, :]
    low = np.tril(np.ones((C, C), dtype=bool))
    return np.where(low, np.exp(np.where(low, diff, 0.0)), 0.0)


def gated_strict_kkt(k, beta, G):
    """S_ri = beta_r exp(G_r - G_i) k_r.k_i for i < r, else 0."""
    k = np.asarray(k, np.float64)
    beta = np.asarray(beta, np.float64)
    C = k.shape[0]
    S = beta[:, None] * decay_matrix(G) * (k @ k.T)
    return S * np.tril(np.ones((C, C)), -1)


def ut_inverse(S):
    """T = (I + S)^-1 for strictly lower-triangular S, by forward substitution
    (row r of (I+S)T = I gives T_r = e_r - sum_{i<r} S_ri T_i)."""
    S = np.asarray(S, np.float64)
    C = S.shape[0]
    T = np.zeros((C, C))
    for r in range(C):
        row = np.zeros(C)
        row[r] = 1.0
        for i in range(r):
            row -= S[r, i] * T[i]
        T[r] = row
    return T


def ut_inverse_ladder(S, base=1):
    """T = (I + S)^-1 by the blockwise doubling ladder of the Pallas-kernel
    page ("Changes", triangular-inversion item): with X the inverse of the
    block-diagonal part at block size b, the inverse at size 2b is
    X - X S_l X, S_l holding only the lower-left b x b block of each 2b x 2b
    diagonal block.  ``base`` > 1 starts from exact inverses of the base x base
    diagonal blocks.  Never forms powers of S.  C must be base * 2^m."""
    S = np.asarray(S, np.float64)
    C = S.shape[0]
    b = int(base)
    if C % b or (C // b) & (C // b - 1):
        raise ValueError("ladder needs C = base * 2^m")
    X = np.zeros((C, C))
    for s in range(0, C, b):
        X[s:s + b, s:s + b] = ut_inverse(S[s:s + b, s:s + b])
    while b < C:
        for s in range(0, C, 2 * b):
            Sl = np.zeros((C, C))
            Sl[s + b:s + 2 * b, s:s + b] = S[s + b:s + 2 * b, s:s + b]
            blk = slice(s, s + 2 * b)
            Xb = X[blk, blk]
            X[blk, blk] = Xb - Xb @ Sl[blk, blk] @ Xb
        b *= 2
    return X


def wy(T, k, v, beta, G):
    """W = T diag(beta e^G) K,  U = T diag(beta) V,  K_g = diag(e^{G_last-G}) K."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    beta = np.asarray(beta, np.float64)
    G = np.asarray(G, np.float64)
    W = T @ ((beta * np.exp(G))[:, None] * k)
    U = T @ (beta[:, None] * v)
    Kg = np.exp(G[-1] - G)[:, None] * k
    return W, U, Kg


def chunk_affine(W, U, Kg, G):
    """The chunk's affine pair: A = e^{G_last} I - K_g^T W,  B = K_g^T U."""
    dk = W.shape[1]
    A = np.exp(G[-1]) * np.eye(dk) - Kg.T @ W
    B = Kg.T @ U
    return A, B


def chunk_step(q, k, v, g, beta, h):
    """One chunk of the chunked form from incoming state h.
    Returns (O [C,d_v], h_end [d_k,d_v], dict of intermediates)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    h = np.asarray(h, np.float64)
    G = decay_cumsum(g)
    S = gated_strict_kkt(k, beta, G)
    T = ut_inverse(S)
    W, U, Kg = wy(T, k, v, beta, G)
    Delta = U - W @ h
    P = (q @ k.T) * decay_matrix(G)          # Gam is already zero above the diagonal
    O = (np.exp(G)[:, None] * q) @ h + P @ Delta
    h_end = np.exp(G[-1]) * h + Kg.T @ Delta
    return O, h_end, dict(G=G, S=S, T=T, W=W, U=U, Kg=Kg, Delta=Delta, P=P)


def compose(p2, p1):
    """(A2, B2) o (A1, B1) = (A2 A1, A2 B1 + B2): apply p1, then p2."""
    A2, B2 = p2
    A1, B1 = p1
    return A2 @ A1, A2 @ B1 + B2


def chunked_forward(q, k, v, g, beta, h0, C):
    """Whole forward by the chunked form, chunk after chunk (fp64).
    q, k [B,T,Hqk,dk]; v [B,T,Hv,dv]; g, beta [B,T,Hv]; h0 [B,Hv,dk,dv] or None.
    T need not be a multiple of C: the last chunk is simply shorter.
    Returns (o [B,T,Hv,dv], hT [B,Hv,dk,dv])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    rep = Hv // Hqk
    o = np.zeros((B, T, Hv, dv))
    hT = np.zeros((B, Hv, dk, dv))
    for b in range(B):
        for hv in range(Hv):
            hq = hv // rep
            h = np.zeros((dk, dv)) if h0 is None else np.asarray(h0[b, hv], np.float64)
            for s in range(0, T, C):
                e = min(s + C, T)
                O, h, _ = chunk_step(q[b, s:e, hq], k[b, s:e, hq], v[b, s:e, hv],
                                     g[b, s:e, hv], beta[b, s:e, hv], h)
                o[b, s:e, hv] = O
            hT[b, hv] = h
    return o, hT
