"""Reference gradients of the per-token gated delta rule, numpy fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring): only the tests may
import this module; the product package never does, and the two share no
code.

The pages give their kernels a backward pass ("Fuse the Gated Delta Net
inter-chunk scan into a Pallas TPU kernel", section "Changes": the scan's
backward walks the chunks in reverse, with the initial and the final state
part of the differentiated chain, and the triangular inverse has an analytic
backward; section "Tests": every gradient, with a non-zero initial state and
a final-state cotangent, is checked against a plain sequential scan).  What
any such backward must produce is the gradient of the per-token rule

    S_t = a_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,   a_t = exp(g_t)
    o_t = S_t^T q_t,                                               S_0 = h0

(the rule of gdn_oracle.c) with respect to q, k, v, g, beta and h0, for
given output cotangents do_t and a final-state cotangent dS_T.  This module
writes that gradient out as reverse-mode differentiation of the rule, one
token at a time from the last to the first -- the definition, with no
chunking, no WY form and no triangular inverse:

    dS <- dS_T (or 0)
    for t = T, ..., 1:
        dS     += q_t do_t^T                 dq_t   = S_t do_t
        r       = k_t^T dS                   p      = k_t^T S_{t-1}     (rows of d_v)
        dv_t    = beta_t r^T                 dbeta_t = r . (v_t - a_t p)
        dg_t    = a_t <dS, S_{t-1} - beta_t k_t p>
        dk_t    = beta_t (dS v_t - a_t (dS p^T + S_{t-1} r^T))
        dS     <- a_t (dS - beta_t k_t r)    (the step's map is symmetric in k)
    dh0 = dS

Value heads that share a query/key head (hv reads head hv // (H_v / H_qk))
add their dq_t and dk_t into that head's.

The chunked form of the same gradients (chunk_step_grad, chunked_bwd: the
forward's chunk quantities differentiated chunk by chunk, the chunks taken
in reverse) is the blueprint of a chunked backward pass; it must equal the
per-token gradients to rounding.

Parity status: pinned by CPU tests (tests/test_oracle_backward.py) against
central finite differences of the forward, against exact identities (o is
linear in q, and jointly linear in (v, h0)), and against the closed form of
the beta = 0 case; the forward it differentiates is checked against
gdn_oracle.c; the chunked form against the per-token one (to ~1e-14) and its
reverse walk against the transposed chunk maps.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    if x is None:
        return None
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, np.float64)


def _heads(q, v):
    Hqk, Hv = q.shape[2], v.shape[2]
    if Hv % Hqk:
        raise ValueError("H_v must be a multiple of H_qk")
    return np.arange(Hv) // (Hv // Hqk)


def states(q, k, v, g, beta, h0=None):
    """The rule run forward: S [T+1, B, H_v, d_k, d_v] (S[0] = h0) and
    o [B, T, H_v, d_v], all fp64."""
    q, k, v, g, beta, h0 = map(_f64, (q, k, v, g, beta, h0))
    B, T, _, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    qh = q[:, :, _heads(q, v)]          # [B,T,Hv,dk]: each value head's query/key rows
    kh = k[:, :, _heads(q, v)]
    S = np.zeros((T + 1, B, Hv, dk, dv))
    if h0 is not None:
        S[0] = h0
    o = np.zeros((B, T, Hv, dv))
    for t in range(T):
        kt, a, bt = kh[:, t], np.exp(g[:, t]), beta[:, t]          # [B,Hv,dk], [B,Hv], [B,Hv]
        p = np.einsum("bhk,bhkv->bhv", kt, S[t])                   # k^T S_{t-1}
        S[t + 1] = a[..., None, None] * (S[t] - bt[..., None, None] * kt[..., :, None] * p[..., None, :]) \
            + bt[..., None, None] * kt[..., :, None] * v[:, t][..., None, :]
        o[:, t] = np.einsum("bhkv,bhk->bhv", S[t + 1], qh[:, t])
    return S, o


def bwd(q, k, v, g, beta, h0=None, do=None, dhT=None):
    """Gradients of L = sum_t <o_t, do_t> + <S_T, dhT> with respect to
    (q, k, v, g, beta, h0), in their shapes, fp64.  do [B,T,H_v,d_v] and dhT
    [B,H_v,d_k,d_v] default to zero.  Returns a dict with keys
    dq, dk, dv, dg, dbeta, dh0."""
    q, k, v, g, beta, h0, do, dhT = map(_f64, (q, k, v, g, beta, h0, do, dhT))
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    hm = _heads(q, v)
    qh, kh = q[:, :, hm], k[:, :, hm]
    S, _ = states(q, k, v, g, beta, h0)
    if do is None:
        do = np.zeros((B, T, Hv, dv))
    dS = np.zeros((B, Hv, dk, dv)) if dhT is None else dhT.copy()
    dqh = np.zeros((B, T, Hv, dk))
    dkh = np.zeros((B, T, Hv, dk))
    dvv = np.zeros((B, T, Hv, dv))
    dg = np.zeros((B, T, Hv))
    db = np.zeros((B, T, Hv))
    for t in range(T - 1, -1, -1):
        St, Sp = S[t + 1], S[t]
        kt, qt, vt, dot = kh[:, t], qh[:, t], v[:, t], do[:, t]
        a, bt = np.exp(g[:, t]), beta[:, t]
        dS = dS + qt[..., :, None] * dot[..., None, :]
        dqh[:, t] = np.einsum("bhkv,bhv->bhk", St, dot)
        r = np.einsum("bhk,bhkv->bhv", kt, dS)
        p = np.einsum("bhk,bhkv->bhv", kt, Sp)
        dvv[:, t] = bt[..., None] * r
        db[:, t] = np.einsum("bhv,bhv->bh", r, vt - a[..., None] * p)
        inner = Sp - bt[..., None, None] * kt[..., :, None] * p[..., None, :]
        dg[:, t] = a * np.einsum("bhkv,bhkv->bh", dS, inner)
        dkh[:, t] = bt[..., None] * (np.einsum("bhkv,bhv->bhk", dS, vt)
                                     - a[..., None] * (np.einsum("bhkv,bhv->bhk", dS, p)
                                                       + np.einsum("bhkv,bhv->bhk", Sp, r)))
        dS = a[..., None, None] * (dS - bt[..., None, None] * kt[..., :, None] * r[..., None, :])
    dq = np.zeros((B, T, Hqk, dk))
    dkk = np.zeros((B, T, Hqk, dk))
    for hv in range(Hv):
        dq[:, :, hm[hv]] += dqh[:, :, hv]
        dkk[:, :, hm[hv]] += dkh[:, :, hv]
    return dict(dq=dq, dk=dkk, dv=dvv, dg=dg, dbeta=db, dh0=dS)


def ut_inverse_grad(T, dT):
    """Cotangent of the strict-lower S for T = (I + S)^-1, given T and the
    cotangent dT: dS = -(T^T dT T^T) restricted to the strict lower triangle
    (S has no other free entries).  This is the analytic backward of the
    triangular inverse that "Fuse the Gated Delta Net inter-chunk scan into a
    Pallas TPU kernel" (section "Changes", triangular-inversion item) states;
    it follows from d(X^-1) = -X^-1 dX X^-1 with X = I + S."""
    T = np.asarray(T, np.float64)
    dT = np.asarray(dT, np.float64)
    return -np.tril(T.T @ dT @ T.T, -1)


def chunk_step_grad(q, k, v, g, beta, h, dO, dh_next):
    """Reverse of one chunk of the chunked form (oracle/chunked.py:
    chunk_step), for one value head: given the chunk's inputs, its incoming
    state h and the cotangents dO [C,d_v] of its outputs and dh_next
    [d_k,d_v] of its outgoing state, the cotangents of q, k, v, g, beta and
    of h.  The chunk's quantities are recomputed from the inputs; each line
    below is the adjoint of one line of the forward, taken in reverse order:

        O      = diag(e^G) Q h + P V'          P = (Q K^T) o Gam (i <= r)
        h_next = e^{G_last} h + K_g^T V'       K_g = diag(e^{G_last - G}) K
        V'     = U - W h
        W      = T diag(beta e^G) K,           U = T diag(beta) V
        T      = (I + S)^-1                    (analytic backward: ut_inverse_grad)
        S      = strict lower of diag(beta) (K K^T o Gam)
        Gam_ri = e^{G_r - G_i} (i <= r),       G = cumsum(g)

    The chunk's backward is what the pages' scan kernel walks in reverse
    ("Fuse the Gated Delta Net inter-chunk scan into a Pallas TPU kernel",
    section "Changes").  Returns a dict dq, dk, dv, dg, dbeta, dh, and the
    reverse walk's chunk-parallel part ddh (the cotangent of h that does not
    pass through dh_next), so that dh = A^T dh_next + ddh with A the chunk's
    state map."""
    from . import chunked

    q, k, v, beta, h, dO, dh_next = (np.asarray(a, np.float64) for a in (q, k, v, beta, h, dO, dh_next))
    O, h_next, it = chunked.chunk_step(q, k, v, g, beta, h)
    G, T, W, U, Kg, Vp, P = it["G"], it["T"], it["W"], it["U"], it["Kg"], it["Delta"], it["P"]
    C = q.shape[0]
    E = np.exp(G)
    Gam = chunked.decay_matrix(G)
    low = np.tril(np.ones((C, C)))
    dG = np.zeros(C)
    # O = diag(E) Q h + P V'
    Qh = q @ h
    dq = E[:, None] * (dO @ h.T)
    dh = q.T @ (E[:, None] * dO)
    dG += E * np.sum(dO * Qh, axis=1)
    dP = (dO @ Vp.T) * low
    dVp = P.T @ dO
    R = q @ k.T
    dR = dP * Gam
    dGam = dP * R
    dq += dR @ k
    dk = dR.T @ q
    # (dh so far and the W path of dVp below form the chunk-parallel term ddh)
    # h_next = e^{G_last} h + K_g^T V'
    eL = np.exp(G[-1])
    dh_walk = eL * dh_next
    dKg = Vp @ dh_next.T
    dVp_walk = Kg @ dh_next
    dG[-1] += eL * np.sum(h * dh_next)
    dscale = np.exp(G[-1] - G)
    dk += dscale[:, None] * dKg
    dd = np.sum(dKg * k, axis=1) * dscale
    dG[-1] += np.sum(dd)
    dG -= dd
    # V' = U - W h
    dVp_all = dVp + dVp_walk
    dU = dVp_all
    dW = -dVp_all @ h.T
    ddh = dh - W.T @ dVp              # chunk-parallel: from dO only
    dh = dh_walk - W.T @ dVp_walk + ddh
    # W = T Wt, U = T Ut
    Wt = (beta * E)[:, None] * k
    Ut = beta[:, None] * v
    dT = dW @ Wt.T + dU @ Ut.T
    dWt = T.T @ dW
    dUt = T.T @ dU
    dk += (beta * E)[:, None] * dWt
    rw = np.sum(dWt * k, axis=1)
    dbeta = rw * E
    dG += beta * E * rw
    dv = beta[:, None] * dUt
    dbeta += np.sum(dUt * v, axis=1)
    # T = (I + S)^-1, S = strict lower of diag(beta)(K K^T o Gam)
    dS = ut_inverse_grad(T, dT)
    Kk = k @ k.T
    dbeta += np.sum(dS * Gam * Kk, axis=1)
    dKk = dS * beta[:, None] * Gam
    dk += (dKk + dKk.T) @ k
    dGam += dS * beta[:, None] * Kk
    # Gam_ri = e^{G_r - G_i} on and below the diagonal
    t = dGam * Gam * low
    dG += np.sum(t, axis=1) - np.sum(t, axis=0)
    # G = cumsum(g)
    dg = np.cumsum(dG[::-1])[::-1]
    return dict(dq=dq, dk=dk, dv=dv, dg=dg, dbeta=dbeta, dh=dh, ddh=ddh)


def chunked_bwd(q, k, v, g, beta, h0=None, do=None, dhT=None, C=64, return_walk=False):
    """The gradients of bwd() computed the chunked way: the forward chunk by
    chunk keeping each chunk's incoming state, then the chunks in reverse,
    each chunk's incoming-state cotangent becoming the previous chunk's
    outgoing one (the reverse walk), with chunk_step_grad per chunk.  The
    last chunk may be shorter.  With ``return_walk`` also returns the
    incoming-state cotangents dh_n [B,H_v,N,d_k,d_v] and the chunk-parallel
    terms ddh_n of the reverse walk."""
    from . import chunked

    q, k, v, g, beta, h0, do, dhT = map(_f64, (q, k, v, g, beta, h0, do, dhT))
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    hm = _heads(q, v)
    if do is None:
        do = np.zeros((B, T, Hv, dv))
    starts = list(range(0, T, C))
    N = len(starts)
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros((B, T, Hv, dv)),
               dg=np.zeros((B, T, Hv)), dbeta=np.zeros((B, T, Hv)), dh0=np.zeros((B, Hv, dk, dv)))
    walk = np.zeros((B, Hv, N, dk, dv))
    par = np.zeros((B, Hv, N, dk, dv))
    for b in range(B):
        for hv in range(Hv):
            hq = hm[hv]
            hs = [np.zeros((dk, dv)) if h0 is None else h0[b, hv].copy()]
            for s in starts:
                e = min(T, s + C)
                _, hn, _ = chunked.chunk_step(q[b, s:e, hq], k[b, s:e, hq], v[b, s:e, hv], g[b, s:e, hv],
                                              beta[b, s:e, hv], hs[-1])
                hs.append(hn)
            dh = np.zeros((dk, dv)) if dhT is None else dhT[b, hv].copy()
            for n in range(N - 1, -1, -1):
                s, e = starts[n], min(T, starts[n] + C)
                r = chunk_step_grad(q[b, s:e, hq], k[b, s:e, hq], v[b, s:e, hv], g[b, s:e, hv],
                                    beta[b, s:e, hv], hs[n], do[b, s:e, hv], dh)
                out["dq"][b, s:e, hq] += r["dq"]
                out["dk"][b, s:e, hq] += r["dk"]
                out["dv"][b, s:e, hv] = r["dv"]
                out["dg"][b, s:e, hv] = r["dg"]
                out["dbeta"][b, s:e, hv] = r["dbeta"]
                dh = r["dh"]
                walk[b, hv, n] = dh
                par[b, hv, n] = r["ddh"]
            out["dh0"][b, hv] = dh
    if return_walk:
        return out, walk, par
    return out
