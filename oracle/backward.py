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

Parity status: pinned by CPU tests (tests/test_oracle_backward.py) against
central finite differences of the forward, against exact identities (o is
linear in q, and jointly linear in (v, h0)), and against the closed form of
the beta = 0 case; the forward it differentiates is checked against
gdn_oracle.c.
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
