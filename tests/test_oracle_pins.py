"""Pins for the fp64 oracle (CPU only).

Each test ties the oracle to something other than itself: a hand-worked
example, closed forms of special cases, invariants of the rule, or an
independent algorithm (the chunked form) that must agree to rounding.
"""
import json
import os

import numpy as np
import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))


def _rand_inputs(B=1, T=40, Hqk=1, Hv=1, dk=8, dv=6, seed=0, h0=True, unit=True):
    rs = np.random.default_rng(seed)
    q = rs.standard_normal((B, T, Hqk, dk)).astype(np.float32)
    k = rs.standard_normal((B, T, Hqk, dk)).astype(np.float32)
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rs.standard_normal((B, T, Hv, dv)).astype(np.float32)
    beta = (1 / (1 + np.exp(-rs.standard_normal((B, T, Hv))))).astype(np.float32)
    g = np.log(1 / (1 + np.exp(-(rs.standard_normal((B, T, Hv)) + 3)))).astype(np.float32)
    hh = (rs.standard_normal((B, Hv, dk, dv)) * 0.5).astype(np.float32) if h0 else None
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=hh)


# ---------------------------------------------------------------------------
# Hand-worked example


def test_golden_hand_example(oracle_lib):
    d = json.load(open(os.path.join(HERE, "golden", "hand_rule_2x2.json")))
    x = d["inputs"]
    f = lambda a: np.asarray(a, np.float32)
    q = f(x["q"])[None, :, None, :]
    k = f(x["k"])[None, :, None, :]
    v = f(x["v"])[None, :, None, :]
    g = f(x["g"])[None, :, None]
    beta = f(x["beta"])[None, :, None]
    o, hT = oracle_lib.fwd(q, k, v, g, beta, None)
    tol = d["tolerance_abs"]
    np.testing.assert_allclose(o[0, :, 0], np.asarray(d["expected"]["o"]), atol=tol, rtol=0)
    np.testing.assert_allclose(hT[0, 0], np.asarray(d["expected"]["h_T"]), atol=tol, rtol=0)


# ---------------------------------------------------------------------------
# Closed forms of special cases


def test_beta_zero_is_pure_decay(oracle_lib):
    x = _rand_inputs(B=2, T=37, Hqk=1, Hv=2, dk=8, dv=6, seed=1)
    x["beta"][:] = 0
    o, hT = oracle_lib.fwd(**x)
    G = np.cumsum(x["g"].astype(np.float64), axis=1)            # [B,T,Hv]
    h0 = x["h0"].astype(np.float64)
    # h_t = e^{G_t} h0  =>  o_t = e^{G_t} h0^T q_t ; h_T = e^{G_T} h0
    for b in range(2):
        for hv in range(2):
            ref_o = np.exp(G[b, :, hv])[:, None] * (x["q"][b, :, 0].astype(np.float64) @ h0[b, hv])
            np.testing.assert_allclose(o[b, :, hv], ref_o, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(hT[b, hv], np.exp(G[b, -1, hv]) * h0[b, hv], rtol=1e-12)


def test_unit_key_overwrite(oracle_lib):
    # g = 0, beta = 1, |k| = 1, q = k:  S_t^T k_t = v_t exactly, so o_t = v_t.
    x = _rand_inputs(T=25, dk=8, dv=5, seed=2)
    # keys with exactly unit norm in fp32: +-1/2 on 4 of the 8 coordinates
    rs = np.random.default_rng(20)
    k = np.zeros((1, 25, 1, 8), np.float32)
    for t in range(25):
        pos = rs.choice(8, 4, replace=False)
        k[0, t, 0, pos] = rs.choice([-0.5, 0.5], 4)
    x["k"] = k
    x["g"][:] = 0
    x["beta"][:] = 1
    x["q"] = x["k"].copy()
    o, _ = oracle_lib.fwd(**x)
    np.testing.assert_allclose(o[0, :, 0], x["v"][0, :, 0].astype(np.float64), atol=1e-12)


def test_basis_keys_reduce_to_scalar_emas(oracle_lib):
    # k_t = e_{i(t)}: the written row follows h <- a(1-beta) h + beta v, the
    # other rows decay by a; with q_t = e_j, o_t reads row j.
    dk, dv, T = 6, 4, 50
    rs = np.random.default_rng(3)
    idx = rs.integers(0, dk, T)
    qi = rs.integers(0, dk, T)
    k = np.zeros((1, T, 1, dk), np.float32)
    k[0, np.arange(T), 0, idx] = 1
    q = np.zeros((1, T, 1, dk), np.float32)
    q[0, np.arange(T), 0, qi] = 1
    v = rs.standard_normal((1, T, 1, dv)).astype(np.float32)
    beta = rs.uniform(0.1, 0.9, (1, T, 1)).astype(np.float32)
    g = -rs.uniform(0.0, 0.3, (1, T, 1)).astype(np.float32)
    h0 = rs.standard_normal((1, 1, dk, dv)).astype(np.float32)
    o, hT = oracle_lib.fwd(q, k, v, g, beta, h0)
    rows = h0[0, 0].astype(np.float64).copy()
    for t in range(T):
        a = np.exp(np.float64(g[0, t, 0]))
        bt = np.float64(beta[0, t, 0])
        for r in range(dk):
            if r == idx[t]:
                rows[r] = a * (1 - bt) * rows[r] + bt * v[0, t, 0].astype(np.float64)
            else:
                rows[r] = a * rows[r]
        np.testing.assert_allclose(o[0, t, 0], rows[qi[t]], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(hT[0, 0], rows, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# Invariants


def test_linear_in_values_and_initial_state(oracle_lib):
    x1 = _rand_inputs(T=30, seed=4)
    x2 = _rand_inputs(T=30, seed=5)
    for key in ("q", "k", "g", "beta"):
        x2[key] = x1[key]
    alpha = np.float32(0.75)
    x3 = dict(x1)
    x3["v"] = (alpha * x1["v"] + x2["v"]).astype(np.float32)
    x3["h0"] = (alpha * x1["h0"] + x2["h0"]).astype(np.float32)
    o1, h1 = oracle_lib.fwd(**x1)
    o2, h2 = oracle_lib.fwd(**x2)
    o3, h3 = oracle_lib.fwd(**x3)
    # x3's fp32 inputs carry their own rounding: compare at fp32-level accuracy
    np.testing.assert_allclose(o3, alpha * o1 + o2, atol=1e-5)
    np.testing.assert_allclose(h3, alpha * h1 + h2, atol=1e-5)


def test_gqa_equals_broadcast_mha(oracle_lib):
    x = _rand_inputs(B=1, T=20, Hqk=2, Hv=4, seed=6)
    o, hT = oracle_lib.fwd(**x)
    rep = dict(x)
    rep["q"] = np.repeat(x["q"], 2, axis=2)
    rep["k"] = np.repeat(x["k"], 2, axis=2)
    o2, h2 = oracle_lib.fwd(**rep)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(hT, h2)


def test_head_permutation_equivariance(oracle_lib):
    x = _rand_inputs(B=1, T=20, Hqk=3, Hv=3, seed=7)
    perm = np.array([2, 0, 1])
    y = dict(x)
    y["q"], y["k"], y["v"] = x["q"][:, :, perm], x["k"][:, :, perm], x["v"][:, :, perm]
    y["g"], y["beta"], y["h0"] = x["g"][:, :, perm], x["beta"][:, :, perm], x["h0"][:, perm]
    o, h = oracle_lib.fwd(**x)
    o2, h2 = oracle_lib.fwd(**y)
    np.testing.assert_array_equal(o[:, :, perm], o2)
    np.testing.assert_array_equal(h[:, perm], h2)


def test_column_and_head_subsets_match_full_run(oracle_lib):
    x = _rand_inputs(B=2, T=19, Hqk=1, Hv=3, dk=8, dv=40, seed=8)
    o, h = oracle_lib.fwd(**x)
    o2, h2 = oracle_lib.fwd(**x, heads=(1, 3), cols=(5, 33))
    np.testing.assert_array_equal(o[:, :, 1:3, 5:33], o2)
    np.testing.assert_array_equal(h[:, 1:3, :, 5:33], h2)


def test_bf16_inputs_are_read_as_rounded_values(oracle_lib):
    x = _rand_inputs(T=16, seed=9)
    xb = dict(x)
    for key in ("q", "k", "v"):
        xb[key] = torch.from_numpy(x[key]).to(torch.bfloat16)
    xr = dict(x)
    for key in ("q", "k", "v"):
        xr[key] = xb[key].float().numpy()
    o, h = oracle_lib.fwd(**xb)
    o2, h2 = oracle_lib.fwd(**xr)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(h, h2)


# ---------------------------------------------------------------------------
# Independent algorithm: the chunked form must reproduce the per-token rule


@pytest.mark.parametrize("C", [1, 2, 8, 16, 48, 64, 128])
def test_chunked_form_equals_per_token_rule(oracle_lib, C):
    x = _rand_inputs(B=1, T=200, Hqk=1, Hv=2, dk=16, dv=12, seed=10 + C)
    o, hT = oracle_lib.fwd(**x)
    oc, hc = oracle_lib.chunked.chunked_forward(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                                x["h0"], C)
    scale = np.sqrt(np.mean(o ** 2))
    assert np.abs(o - oc).max() <= 1e-12 * scale
    assert np.abs(hT - hc).max() <= 1e-12 * np.sqrt(np.mean(hT ** 2))


def test_chunk_of_one_token_is_the_rule(oracle_lib):
    # C = 1: A = e^g (I - beta k k^T), B = beta k v^T
    ch = oracle_lib.chunked
    rs = np.random.default_rng(11)
    k = rs.standard_normal((1, 5))
    v = rs.standard_normal((1, 3))
    g, beta = np.array([-0.3]), np.array([0.7])
    G = ch.decay_cumsum(g)
    T = ch.ut_inverse(ch.gated_strict_kkt(k, beta, G))
    W, U, Kg = ch.wy(T, k, v, beta, G)
    A, Bm = ch.chunk_affine(W, U, Kg, G)
    np.testing.assert_allclose(A, np.exp(-0.3) * (np.eye(5) - 0.7 * np.outer(k[0], k[0])),
                               rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(Bm, 0.7 * np.outer(k[0], v[0]), rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------------------
# The UT transform (I+S)^-1


def _strict(S):
    return np.tril(S, -1)


@pytest.mark.parametrize("kind", ["random", "ones", "gauss_unnormalised"])
@pytest.mark.parametrize("C", [16, 64, 128])
def test_ut_inverse_residual_and_ladder(oracle_lib, kind, C):
    ch = oracle_lib.chunked
    rs = np.random.default_rng(C)
    if kind == "ones":
        S = _strict(np.ones((C, C)))
    else:
        k = rs.standard_normal((C, 32))
        if kind == "random":
            k /= np.linalg.norm(k, axis=1, keepdims=True)
        beta = 1 / (1 + np.exp(-rs.standard_normal(C)))
        g = np.log(1 / (1 + np.exp(-(rs.standard_normal(C) + 3))))
        S = ch.gated_strict_kkt(k, beta, ch.decay_cumsum(g))
    T = ch.ut_inverse(S)
    I = np.eye(C)
    scale = max(1.0, np.abs(T).max())
    assert np.isfinite(T).all()
    assert np.abs((I + S) @ T - I).max() <= 1e-10 * scale * max(1.0, np.abs(S).max())
    for base in (1, 16):
        Tl = ch.ut_inverse_ladder(S, base=base)
        assert np.isfinite(Tl).all()
        assert np.abs(Tl - T).max() <= 1e-9 * scale
    if kind == "ones":
        # (I + strict ones)^-1 = I - (first subdiagonal of ones)
        np.testing.assert_array_equal(T, I - np.eye(C, k=-1))


def test_ut_inverse_single_subdiagonal_closed_form(oracle_lib):
    ch = oracle_lib.chunked
    C = 12
    rs = np.random.default_rng(12)
    s = rs.uniform(-1.5, 1.5, C)
    S = np.zeros((C, C))
    for r in range(1, C):
        S[r, r - 1] = s[r]
    T = ch.ut_inverse(S)
    for r in range(C):
        for i in range(C):
            ref = 0.0 if i > r else (-1.0) ** (r - i) * np.prod(s[i + 1:r + 1])
            assert abs(T[r, i] - ref) <= 1e-13 * max(1.0, abs(ref))
    np.testing.assert_allclose(ch.ut_inverse_ladder(S[:8, :8], base=1),
                               ch.ut_inverse(S[:8, :8]), rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------------------
# The affine inter-chunk step and its composition


def test_affine_step_equals_per_token_walk(oracle_lib):
    ch = oracle_lib.chunked
    x = _rand_inputs(T=64, dk=16, dv=12, seed=13)
    q, k, v = x["q"][0, :, 0], x["k"][0, :, 0], x["v"][0, :, 0]
    g, beta, h = x["g"][0, :, 0], x["beta"][0, :, 0], x["h0"][0, 0]
    G = ch.decay_cumsum(g)
    T = ch.ut_inverse(ch.gated_strict_kkt(k, beta, G))
    W, U, Kg = ch.wy(T, k, v, beta, G)
    A, Bm = ch.chunk_affine(W, U, Kg, G)
    _, hT = oracle_lib.fwd(**x)
    np.testing.assert_allclose(A @ h.astype(np.float64) + Bm, hT[0, 0], rtol=1e-11, atol=1e-13)
    # B alone is the walk from h = 0
    x0 = dict(x)
    x0["h0"] = None
    _, hT0 = oracle_lib.fwd(**x0)
    np.testing.assert_allclose(Bm, hT0[0, 0], rtol=1e-11, atol=1e-13)


def test_fold_equals_chunk_affine_pairs(oracle_lib):
    ch = oracle_lib.chunked
    x = _rand_inputs(T=96, Hqk=1, Hv=2, dk=16, dv=12, seed=14)
    A, Bm = oracle_lib.fold(x["k"], x["v"], x["g"], x["beta"], n_groups=3)
    for hv in range(2):
        for j in range(3):
            s = slice(32 * j, 32 * (j + 1))
            k, v = x["k"][0, s, 0], x["v"][0, s, hv]
            g, beta = x["g"][0, s, hv], x["beta"][0, s, hv]
            G = ch.decay_cumsum(g)
            T = ch.ut_inverse(ch.gated_strict_kkt(k, beta, G))
            W, U, Kg = ch.wy(T, k, v, beta, G)
            Ac, Bc = ch.chunk_affine(W, U, Kg, G)
            np.testing.assert_allclose(A[0, hv, j], Ac, rtol=1e-11, atol=1e-13)
            np.testing.assert_allclose(Bm[0, hv, j], Bc, rtol=1e-11, atol=1e-13)


def test_sequential_fold_equals_tree_composition(oracle_lib):
    ch = oracle_lib.chunked
    x = _rand_inputs(T=128, dk=8, dv=6, seed=15)
    A, Bm = oracle_lib.fold(x["k"], x["v"], x["g"], x["beta"], n_groups=8)
    pairs = [(A[0, 0, j], Bm[0, 0, j]) for j in range(8)]
    # left-to-right sequential composition
    seq = pairs[0]
    for p in pairs[1:]:
        seq = ch.compose(p, seq)
    # balanced tree composition
    level = pairs
    while len(level) > 1:
        level = [ch.compose(level[i + 1], level[i]) for i in range(0, len(level), 2)]
    np.testing.assert_allclose(level[0][0], seq[0], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(level[0][1], seq[1], rtol=1e-12, atol=1e-15)
    # and the whole-sequence fold is one pair
    A1, B1 = oracle_lib.fold(x["k"], x["v"], x["g"], x["beta"], n_groups=1)
    np.testing.assert_allclose(A1[0, 0, 0], seq[0], rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(B1[0, 0, 0], seq[1], rtol=1e-10, atol=1e-14)


def test_prefix_reproduces_states_at_group_boundaries(oracle_lib):
    x = _rand_inputs(B=1, T=120, Hqk=1, Hv=2, dk=8, dv=6, seed=16)
    ng, L = 6, 20
    A, Bm = oracle_lib.fold(x["k"], x["v"], x["g"], x["beta"], n_groups=ng)
    h_in, h_fin = oracle_lib.prefix(A.reshape(2, ng, 8, 8), Bm.reshape(2, ng, 8, 6),
                                    x["h0"].reshape(2, 8, 6))
    for j in range(ng + 1):
        if j == 0:
            ref = x["h0"][0].astype(np.float64)
        else:
            y = {key: (val[:, :j * L] if key not in ("h0",) else val) for key, val in x.items()}
            _, ref = oracle_lib.fwd(**y)
            ref = ref[0]
        got = h_in[:, j] if j < ng else h_fin
        # the pairs pass through fp32 on their way into the prefix
        np.testing.assert_allclose(got, ref, rtol=0, atol=2e-5 * max(1.0, np.abs(ref).max()))


def test_state_threading_split_run(oracle_lib):
    x = _rand_inputs(B=1, T=90, Hqk=1, Hv=1, seed=17)
    o, hT = oracle_lib.fwd(**x)
    T1 = 37
    a = {key: (val[:, :T1] if key != "h0" else val) for key, val in x.items()}
    oa, ha = oracle_lib.fwd(**a)
    b = {key: (val[:, T1:] if key != "h0" else val) for key, val in x.items()}
    b["h0"] = ha.astype(np.float32)
    ob, hb = oracle_lib.fwd(**b)
    np.testing.assert_array_equal(oa, o[:, :T1])
    np.testing.assert_allclose(ob, o[:, T1:], atol=1e-6)
    np.testing.assert_allclose(hb, hT, atol=1e-6)


def test_negative_control_zeroed_incoming_states_fail(oracle_lib):
    # Replaying each group from a zero state (the isolated-shard mistake)
    # must miss the tolerance by a wide margin, most of all with weak decay,
    # where a group's affine map stays far from zero.
    x = _rand_inputs(B=1, T=256, Hqk=1, Hv=1, dk=16, dv=16, seed=18)
    x["g"][:] = 0
    x["beta"] *= 0.1
    o, hT = oracle_lib.fwd(**x)
    L, ng = 64, 4
    bad = np.empty_like(o)
    h = None
    for j in range(ng):
        y = {key: (val[:, j * L:(j + 1) * L] if key != "h0" else None) for key, val in x.items()}
        bad[:, j * L:(j + 1) * L], h = oracle_lib.fwd(**y)
    rms = np.sqrt(np.mean(o ** 2))
    assert np.abs(bad - o).max() > 10 * 2e-2 * rms
    assert np.abs(h - hT).max() > 10 * 2e-2 * np.sqrt(np.mean(hT ** 2))
