"""Pins for the fp64 reference gradients of the rule (CPU only).

oracle/backward.py differentiates the per-token rule by hand; these tests tie
it to the forward (central finite differences), to exact identities of the
rule, and to the closed form of a special case; and the triangular inverse's
analytic backward to central differences of the inverse itself.
"""
import numpy as np
import pytest

from oracle import backward as bw


def _inputs(B=1, T=7, Hqk=1, Hv=2, dk=4, dv=3, seed=0, h0=True, beta_zero=False):
    rs = np.random.default_rng(seed)
    q = rs.standard_normal((B, T, Hqk, dk))
    k = rs.standard_normal((B, T, Hqk, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rs.standard_normal((B, T, Hv, dv))
    beta = 1 / (1 + np.exp(-rs.standard_normal((B, T, Hv))))
    if beta_zero:
        beta[:] = 0
    g = np.log(1 / (1 + np.exp(-(rs.standard_normal((B, T, Hv)) + 2))))
    h0 = rs.standard_normal((B, Hv, dk, dv)) * 0.5 if h0 else None
    do = rs.standard_normal((B, T, Hv, dv))
    dhT = rs.standard_normal((B, Hv, dk, dv))
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0), do, dhT


def _loss(x, do, dhT):
    S, o = bw.states(**x)
    return float(np.sum(o * do) + np.sum(S[-1] * dhT))


def test_forward_matches_the_c_oracle(oracle_lib):
    # the forward that the gradients differentiate is the rule of gdn_oracle.c
    x, _, _ = _inputs(B=2, T=33, Hqk=2, Hv=4, dk=8, dv=6, seed=1)
    xf = {kk: vv.astype(np.float32) for kk, vv in x.items()}
    xd = {kk: vv.astype(np.float64) for kk, vv in xf.items()}   # the same rounded inputs in fp64
    S, o = bw.states(**xd)
    o_c, hT_c = oracle_lib.fwd(**xf)
    np.testing.assert_allclose(o, o_c, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S[-1], hT_c, rtol=0, atol=1e-12)


@pytest.mark.parametrize("Hqk,Hv", [(1, 1), (1, 2), (2, 2)])
def test_gradients_match_central_differences(Hqk, Hv):
    # every element of every input, perturbed by +-eps in fp64: the central
    # difference of L = sum <o, do> + <S_T, dS_T> (error O(eps^2) ~ 1e-12
    # relative) against the hand-written reverse pass; with two value heads
    # per query/key head the shared dq and dk are sums over both
    x, do, dhT = _inputs(Hqk=Hqk, Hv=Hv, seed=2 + Hv)
    grads = bw.bwd(**x, do=do, dhT=dhT)
    eps = 1e-6
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"), ("h0", "dh0")):
        base = x[name]
        fd = np.zeros_like(base)
        for i in np.ndindex(base.shape):
            keep = base[i]
            base[i] = keep + eps
            lp = _loss(x, do, dhT)
            base[i] = keep - eps
            lm = _loss(x, do, dhT)
            base[i] = keep
            fd[i] = (lp - lm) / (2 * eps)
        err = np.abs(fd - grads[gname]).max()
        assert err <= 1e-7 * max(1.0, np.abs(fd).max()), f"{gname}: {err:.3e}"


def test_gradients_wrt_q_and_values_follow_linearity():
    # o is linear in q, and (o, S_T) jointly linear in (v, h0) for fixed k, g,
    # beta: Euler's identity for degree-1 homogeneous maps gives
    # sum q.dq = sum o.do (with dS_T = 0) and sum v.dv + <h0, dh0> = L exactly
    x, do, dhT = _inputs(B=2, T=40, Hqk=2, Hv=4, dk=16, dv=16, seed=7)
    S, o = bw.states(**x)
    L_o = float(np.sum(o * do))
    gq = bw.bwd(**x, do=do)
    assert abs(np.sum(x["q"] * gq["dq"]) - L_o) <= 1e-10 * max(1.0, abs(L_o))
    gv = bw.bwd(**x, do=do, dhT=dhT)
    L = L_o + float(np.sum(S[-1] * dhT))
    lhs = np.sum(x["v"] * gv["dv"]) + np.sum(x["h0"] * gv["dh0"])
    assert abs(lhs - L) <= 1e-10 * max(1.0, abs(L))


def test_beta_zero_closed_form():
    # beta = 0: S_t = e^{G_t} h0 with G_t = g_1 + ... + g_t, o_t = S_t^T q_t.
    # Then dq_t = S_t do_t, dk = dv = 0, dh0 = sum_t e^{G_t} q_t do_t^T +
    # e^{G_T} dS_T and dg_t = sum_{tau >= t} <q_tau do_tau^T, S_tau> + <dS_T, S_T>
    x, do, dhT = _inputs(B=1, T=9, Hqk=1, Hv=2, dk=5, dv=4, seed=11, beta_zero=True)
    gr = bw.bwd(**x, do=do, dhT=dhT)
    G = np.cumsum(x["g"], axis=1)                                  # [B,T,Hv]
    St = np.exp(G)[..., None, None] * x["h0"][:, None]            # [B,T,Hv,dk,dv]
    qh = x["q"][:, :, [0, 0]]
    np.testing.assert_allclose(gr["dq"][:, :, 0], np.einsum("bthkv,bthv->btk", St, do), rtol=1e-12, atol=1e-12)
    assert np.abs(gr["dk"]).max() == 0 and np.abs(gr["dv"]).max() == 0
    dh0 = np.einsum("bth,bthk,bthv->bhkv", np.exp(G), qh, do) + np.exp(G[:, -1])[..., None, None] * dhT
    np.testing.assert_allclose(gr["dh0"], dh0, rtol=1e-12, atol=1e-12)
    per_t = np.einsum("bthk,bthv,bthkv->bth", qh, do, St)          # <q_t do_t^T, S_t>
    tail = np.cumsum(per_t[:, ::-1], axis=1)[:, ::-1]              # sum over tau >= t
    dg = tail + np.einsum("bhkv,bhkv->bh", dhT, St[:, -1])[:, None, :]
    np.testing.assert_allclose(gr["dg"], dg, rtol=1e-12, atol=1e-12)


def test_zero_cotangents_give_zero_gradients():
    x, do, dhT = _inputs(seed=5)
    gr = bw.bwd(**x)
    assert all(np.abs(vv).max() == 0 for vv in gr.values())


@pytest.mark.parametrize("C", [8, 32])
def test_ut_inverse_grad_matches_central_differences(C):
    # the analytic backward of the triangular inverse against central
    # differences of the forward-substitution inverse, entry by entry over the
    # strict lower triangle (the only free entries of S)
    from oracle import chunked

    rs = np.random.default_rng(C)
    k = rs.standard_normal((C, 6))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    beta = 1 / (1 + np.exp(-rs.standard_normal(C)))
    G = np.cumsum(np.log(1 / (1 + np.exp(-(rs.standard_normal(C) + 3)))))
    S = chunked.gated_strict_kkt(k, beta, G)
    dT = rs.standard_normal((C, C))
    T = chunked.ut_inverse(S)
    dS = bw.ut_inverse_grad(T, dT)
    eps = 1e-6
    fd = np.zeros_like(S)
    for i in range(C):
        for j in range(i):
            Sp, Sm = S.copy(), S.copy()
            Sp[i, j] += eps
            Sm[i, j] -= eps
            fd[i, j] = np.sum((chunked.ut_inverse(Sp) - chunked.ut_inverse(Sm)) * dT) / (2 * eps)
    assert np.abs(np.triu(dS)).max() == 0
    assert np.abs(fd - dS).max() <= 1e-7 * max(1.0, np.abs(fd).max())


@pytest.mark.parametrize("C,T,Hqk,Hv,h0", [(1, 6, 1, 1, True), (4, 21, 1, 2, True), (16, 48, 2, 4, False),
                                           (16, 37, 1, 3, True)])
def test_chunked_backward_equals_per_token(C, T, Hqk, Hv, h0):
    # two independent derivations of the same gradients: the per-token reverse
    # pass and the chunked one (WY form, triangular inverse and its analytic
    # backward, reverse walk over chunks; a shorter last chunk when C does not
    # divide T)
    x, do, dhT = _inputs(B=2, T=T, Hqk=Hqk, Hv=Hv, dk=6, dv=5, seed=C + T, h0=h0)
    a = bw.bwd(**x, do=do, dhT=dhT)
    c = bw.chunked_bwd(**x, do=do, dhT=dhT, C=C)
    for kk in a:
        assert np.abs(a[kk] - c[kk]).max() <= 1e-12 * max(1.0, np.abs(a[kk]).max()), kk


def test_reverse_walk_is_the_transposed_chunk_map():
    # the cotangent of each chunk's incoming state is A_n^T (that of its
    # outgoing state) + a term that depends on the chunk's own outputs only,
    # A_n the chunk's state map e^{G_last} I - K_g^T W
    from oracle import chunked

    C = 8
    x, do, dhT = _inputs(B=1, T=5 * C, Hqk=1, Hv=1, dk=6, dv=5, seed=3)
    _, walk, par = bw.chunked_bwd(**x, do=do, dhT=dhT, C=C, return_walk=True)
    nxt = dhT[0, 0]
    for n in range(4, -1, -1):
        s = slice(n * C, (n + 1) * C)
        G = chunked.decay_cumsum(x["g"][0, s, 0])
        T = chunked.ut_inverse(chunked.gated_strict_kkt(x["k"][0, s, 0], x["beta"][0, s, 0], G))
        W, U, Kg = chunked.wy(T, x["k"][0, s, 0], x["v"][0, s, 0], x["beta"][0, s, 0], G)
        A, _ = chunked.chunk_affine(W, U, Kg, G)
        np.testing.assert_allclose(walk[0, 0, n], A.T @ nxt + par[0, 0, n], rtol=0, atol=1e-12)
        nxt = walk[0, 0, n]
    # with no output cotangent the walk is the transposed maps alone
    _, walk0, par0 = bw.chunked_bwd(**x, dhT=dhT, C=C, return_walk=True)
    assert np.abs(par0).max() == 0
