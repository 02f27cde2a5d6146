"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances: max-abs error <= 1e-4 * RMS for fp32 inputs and <= 2e-2 * RMS for
bf16 inputs, on o and on h_T.  Each tensor is gated against the RMS of the
oracle's own tensor and also against RMS(o) (the two readings of "RMS(o)"
for h_T); both must pass.  Intermediate steps (decay cumsum, UT inverse, W,
U, fold pairs, prefix) are checked against the oracle's fp64 values of the
same quantities.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module")
def gdn():
    import linear_attention_rnn_gdn_amd as g

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.lib()
    return g


def _rms(x):
    return float(np.sqrt(np.mean(np.asarray(x, np.float64) ** 2)))


def _err(got, ref):
    return float(np.abs(np.asarray(got, np.float64) - ref).max())


def _check(name, got, ref, tol, rms_o):
    e = _err(got, ref)
    lim = tol * min(_rms(ref), rms_o)
    print(f"  {name}: max-abs {e:.3e}  limit {lim:.3e}  (rel to RMS {e / max(_rms(ref), 1e-30):.2e})",
          flush=True)
    assert e <= lim, f"{name}: max-abs error {e:.3e} > {lim:.3e}"


def _cpu(x):
    return None if x is None else x.detach().cpu()


def _run_and_compare(gdn, w, x, heads=None, cols=None, o_dtype=torch.float32, n_groups=None):
    ng = w.n_groups if n_groups is None else n_groups
    o, hT = gdn.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], chunk=w.chunk,
                          n_groups=ng, o_dtype=o_dtype)
    torch.cuda.synchronize()
    hl, hh = heads if heads else (0, w.Hv)
    cl, ch = cols if cols else (0, w.dv)
    if heads or cols:
        hq_lo = hl // (w.Hv // w.Hqk)
        hq_hi = (hh - 1) // (w.Hv // w.Hqk) + 1
        rep = w.Hv // w.Hqk
        # the oracle sees only the needed heads: re-index value heads from 0
        sub = dict(
            q=_cpu(x["q"][:, :, hq_lo:hq_hi]), k=_cpu(x["k"][:, :, hq_lo:hq_hi]),
            v=_cpu(x["v"][:, :, hq_lo * rep:hq_hi * rep]),
            g=_cpu(x["g"][:, :, hq_lo * rep:hq_hi * rep]),
            beta=_cpu(x["beta"][:, :, hq_lo * rep:hq_hi * rep]),
            h0=_cpu(x["h0"][:, hq_lo * rep:hq_hi * rep]) if x["h0"] is not None else None)
        o_ref, h_ref = oracle.fwd(**sub, heads=(hl - hq_lo * rep, hh - hq_lo * rep), cols=(cl, ch))
    else:
        o_ref, h_ref = oracle.fwd(**{kk: _cpu(vv) for kk, vv in x.items()})
    o_got = o[:, :, hl:hh, cl:ch].float().cpu().numpy()
    h_got = hT[:, hl:hh, :, cl:ch].cpu().numpy()
    return o_got, h_got, o_ref, h_ref


# ---------------------------------------------------------------------------
# rows a1-a4: decay cumsum, UT inverse, W, U


@pytest.mark.parametrize("dtype,C", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_chunk_transform_matches_oracle(gdn, dtype, C):
    w = WORKLOADS["tiny"].replace(T=4 * C, Hqk=1, Hv=2, chunk=C, dtype=dtype)
    x = make_inputs(w, device="cuda", seed=7)
    G, Tm, W, U = gdn.chunk_transform(x["k"], x["v"], x["g"], x["beta"], chunk=C, want_T=True)
    torch.cuda.synchronize()
    ch = oracle.chunked
    k = x["k"].float().cpu().numpy()
    v = x["v"].float().cpu().numpy()
    g = x["g"].cpu().numpy()
    beta = x["beta"].cpu().numpy()
    tol = 1e-5 if dtype == "f32" else 2e-4
    for hv in range(2):
        for n in range(4):
            s = slice(n * C, (n + 1) * C)
            Gr = ch.decay_cumsum(g[0, s, hv])
            S = ch.gated_strict_kkt(k[0, s, 0], beta[0, s, hv], Gr)
            Tr = ch.ut_inverse(S)
            Wr, Ur, _ = ch.wy(Tr, k[0, s, 0], v[0, s, hv], beta[0, s, hv], Gr)
            assert _err(G[0, hv, n].cpu().numpy(), Gr) <= 1e-5 * max(1, np.abs(Gr).max())
            assert _err(Tm[0, hv, n].cpu().numpy(), Tr) <= tol * max(1, np.abs(Tr).max())
            assert _err(W[0, hv, n].cpu().numpy(), Wr) <= tol * max(_rms(Wr), 1e-3) * 10
            assert _err(U[0, hv, n].cpu().numpy(), Ur) <= tol * max(_rms(Ur), 1e-3) * 10
            # (I + S) T = I on the GPU's T
            res = (np.eye(C) + S) @ Tm[0, hv, n].cpu().numpy().astype(np.float64) - np.eye(C)
            assert np.abs(res).max() <= tol * 10


def test_ut_inverse_all_ones_gram(gdn):
    # unit keys all equal, beta = 1, g = 0: S = strict-lower ones, T = I - subdiagonal
    C = 128
    w = WORKLOADS["tiny"].replace(T=C, Hqk=1, Hv=1, chunk=C, dtype="bf16")
    x = make_inputs(w, device="cuda", seed=1)
    e = torch.zeros(128, device="cuda")
    e[3] = 1.0
    x["k"][:] = e.to(torch.bfloat16)
    x["beta"][:] = 1.0
    x["g"][:] = 0.0
    _, Tm, _, _ = gdn.chunk_transform(x["k"], x["v"], x["g"], x["beta"], chunk=C, want_T=True)
    ref = np.eye(C) - np.eye(C, k=-1)
    assert _err(Tm[0, 0, 0].cpu().numpy(), ref) <= 1e-5


# ---------------------------------------------------------------------------
# rows a5-a6 end to end, single walk


@pytest.mark.parametrize("name", ["tiny", "qwen3next_8b_layer"])
def test_forward_full_size(gdn, name):
    w = WORKLOADS[name]
    x = make_inputs(w, device="cuda")
    o, h, o_ref, h_ref = _run_and_compare(gdn, w, x)
    ro = _rms(o_ref)
    _check("o", o, o_ref, TOL[w.dtype], ro)
    _check("h_T", h, h_ref, TOL[w.dtype], ro)


def test_forward_dense_layer_full_size(gdn):
    w = WORKLOADS["dense_d4096_layer"]
    x = make_inputs(w, device="cuda")
    o, h, o_ref, h_ref = _run_and_compare(gdn, w, x)
    ro = _rms(o_ref)
    _check("o", o, o_ref, TOL[w.dtype], ro)
    _check("h_T", h, h_ref, TOL[w.dtype], ro)


@pytest.mark.parametrize("dtype,C,T,Hqk,Hv,h0", [
    ("bf16", 64, 640, 2, 4, 0.02),
    ("bf16", 128, 128, 1, 1, 0.0),        # a single chunk
    ("f32", 64, 64 * 7, 1, 3, 0.5),        # odd chunk count, strong h0
    ("bf16", 128, 128 * 9, 3, 6, 0.1),
])
def test_forward_small_shapes(gdn, dtype, C, T, Hqk, Hv, h0):
    w = WORKLOADS["tiny"].replace(T=T, Hqk=Hqk, Hv=Hv, chunk=C, dtype=dtype, h0_std=h0, B=2)
    x = make_inputs(w, device="cuda", seed=T + Hv)
    o, h, o_ref, h_ref = _run_and_compare(gdn, w, x)
    ro = _rms(o_ref)
    _check("o", o, o_ref, TOL[dtype], ro)
    _check("h_T", h, h_ref, TOL[dtype], ro)


@pytest.mark.parametrize("case", ["beta0", "overwrite", "strong_decay", "resets", "large_scale"])
@pytest.mark.parametrize("C", [64, 128])
def test_degenerate_inputs(gdn, case, C):
    # the rule's special cases, against the fp64 oracle at the bf16 bar:
    #   beta0         beta = 0: no writes, the state only decays (o = e^G Q h0)
    #   overwrite     g = 0, beta = 1, one-hot keys repeating within a chunk:
    #                 each write replaces the row of its key (S has unit entries)
    #   strong_decay  g = -20 per token: e^G underflows to 0 inside a chunk
    #   resets        usual g, with g = -60 every 37th token (state wiped)
    #   large_scale   v and h0 scaled by 1e3 (o and h_T scale with them)
    w = WORKLOADS["tiny"].replace(T=C * 6, Hqk=1, Hv=2, chunk=C, dtype="bf16", h0_std=0.5)
    x = make_inputs(w, device="cuda", seed=11 + C)
    T = w.T
    if case == "beta0":
        x["beta"] = torch.zeros_like(x["beta"])
    elif case == "overwrite":
        x["g"] = torch.zeros_like(x["g"])
        x["beta"] = torch.ones_like(x["beta"])
        idx = (torch.arange(T, device="cuda") * 5) % 24           # 24 distinct keys
        k = torch.zeros_like(x["k"])
        k[0, torch.arange(T, device="cuda"), :, idx] = 1.0
        x["k"] = k
    elif case == "strong_decay":
        x["g"] = torch.full_like(x["g"], -20.0)
    elif case == "resets":
        g = x["g"].clone()
        g[:, ::37] = -60.0
        x["g"] = g
    elif case == "large_scale":
        x["v"] = (x["v"].float() * 1e3).to(torch.bfloat16)
        x["h0"] = x["h0"] * 1e3
    o, h, o_ref, h_ref = _run_and_compare(gdn, w, x)
    assert np.isfinite(o).all() and np.isfinite(h).all()
    ro = _rms(o_ref)
    _check("o", o, o_ref, TOL["bf16"], ro)
    _check("h_T", h, h_ref, TOL["bf16"], ro)


def test_bf16_output(gdn):
    # a bf16 o carries its own rounding (half an ulp of |o|) on top of the
    # computation error
    w = WORKLOADS["tiny"].replace(T=1024, Hqk=2, Hv=4, chunk=128, dtype="bf16", h0_std=0.02)
    x = make_inputs(w, device="cuda", seed=3)
    o, h, o_ref, h_ref = _run_and_compare(gdn, w, x, o_dtype=torch.bfloat16)
    ro = _rms(o_ref)
    bound = 2e-2 * ro + np.abs(o_ref) * 2.0 ** -8
    assert (np.abs(o - o_ref) <= bound).all()
    _check("h_T", h, h_ref, 2e-2, ro)


@pytest.mark.parametrize("dtype,C,B,Hqk,Hv,T", [
    ("bf16", 128, 4, 16, 32, 1000),     # 128 walks: one state slice per wave
    ("bf16", 64, 8, 8, 16, 64 * 5),
    ("f32", 64, 6, 8, 24, 64 * 4 - 9),
    ("bf16", 128, 5, 17, 51, 300),      # 255 walks, partial last chunk
    ("bf16", 128, 8, 16, 32, 1000),     # 256 walks: two state slices per wave
    ("bf16", 64, 16, 8, 16, 64 * 3),    # 256 walks at C = 64
    ("f32", 64, 8, 8, 32, 64 * 3 - 5),  # 256 walks, fp32, partial last chunk
])
def test_walk_with_outputs_bf16_output(gdn, dtype, C, B, Hqk, Hv, T):
    # 128 walks or more: the walk forms the outputs itself (walk_out_kernel),
    # from 256 walks on with two state slices per wave.  A bf16 o is the
    # fp32-o call's values rounded once, bit for bit; the fp32 o within the bar
    w = WORKLOADS["tiny"].replace(T=T, B=B, Hqk=Hqk, Hv=Hv, chunk=C, dtype=dtype, h0_std=0.05)
    x = make_inputs(w, device="cuda", seed=B * Hv + T)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    o32, h32 = gdn.chunk_fwd(*args, chunk=C)
    o16, h16 = gdn.chunk_fwd(*args, chunk=C, o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16)) and torch.equal(h16, h32)
    o_ref, h_ref = oracle.fwd(**{kk: _cpu(vv) for kk, vv in x.items()})
    ro = _rms(o_ref)
    _check("o", o32.cpu().numpy(), o_ref, TOL[dtype], ro)
    _check("h_T", h32.cpu().numpy(), h_ref, TOL[dtype], ro)


def test_empty_sequence_returns_initial_state(gdn):
    w = WORKLOADS["tiny"].replace(T=0, dtype="bf16", chunk=128, h0_std=0.3)
    x = make_inputs(w, device="cuda", seed=5)
    o, hT = gdn.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], chunk=128)
    torch.cuda.synchronize()
    assert o.numel() == 0
    assert torch.equal(hT, x["h0"])
    o, hT = gdn.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], None, chunk=128)
    torch.cuda.synchronize()
    assert torch.count_nonzero(hT) == 0


def test_gqa_equals_broadcast_mha_on_gpu(gdn):
    w = WORKLOADS["tiny"].replace(T=512, Hqk=2, Hv=4, chunk=128, dtype="bf16", h0_std=0.02)
    x = make_inputs(w, device="cuda", seed=9)
    o1, h1 = gdn.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], chunk=128)
    q2 = x["q"].repeat_interleave(2, dim=2).contiguous()
    k2 = x["k"].repeat_interleave(2, dim=2).contiguous()
    o2, h2 = gdn.chunk_fwd(q2, k2, x["v"], x["g"], x["beta"], x["h0"], chunk=128)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_run_to_run_bitwise_determinism(gdn):
    w = WORKLOADS["qwen3next_8b_layer"]
    x = make_inputs(w, device="cuda")
    a = gdn.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], chunk=128)
    b = gdn.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], chunk=128)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("C,N,ng,tail", [(64, 16, 0, 0), (128, 32, 0, 0), (128, 16, 4, 0), (128, 16, 4, 37)])
def test_stages_one_by_one_equal_one_call(gdn, C, N, ng, tail):
    # gdn_chunk_fwd_stages issued one stage per call on one stream (the
    # per-kernel timing path of bench.py) must equal one gdn_chunk_fwd call
    # bit for bit: the stages communicate only through the workspace (also
    # with a partial last chunk: `tail` tokens short)
    w = WORKLOADS["tiny"].replace(T=C * N - tail, Hqk=2, Hv=4, chunk=C, dtype="bf16", h0_std=0.05)
    x = make_inputs(w, device="cuda", seed=N + ng)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    o1, h1 = gdn.chunk_fwd(*args, chunk=C, n_groups=ng)
    shape = gdn.make_shape(w.B, w.T, w.Hqk, w.Hv, 128, 128, C, ng, x["k"].dtype, torch.float32)
    ws = torch.empty(gdn.workspace_size(shape), dtype=torch.uint8, device="cuda")
    o2, h2 = torch.empty_like(o1), torch.empty_like(h1)
    stages = [gdn.STAGE_PREP] + ([gdn.STAGE_FOLD, gdn.STAGE_PREFIX] if ng > 1 else []) + \
        [gdn.STAGE_WALK, gdn.STAGE_OUT]
    for st in stages:
        gdn.chunk_fwd(*args, chunk=C, n_groups=ng, workspace=ws, out=o2, final_state=h2, stages=st)
    o3, h3 = gdn.chunk_fwd(*args, chunk=C, n_groups=ng, output_final_state=False)
    torch.cuda.synchronize()
    assert h3 is None
    assert torch.equal(o1, o2) and torch.equal(h1, h2) and torch.equal(o1, o3)


@pytest.mark.parametrize("ng", [0, 4])
def test_timed_call_equals_plain_call(gdn, ng):
    # gdn_chunk_fwd_timed (bench.py's per-kernel timing) computes what
    # gdn_chunk_fwd does, bit for bit, and every timed stage's events bound a
    # positive duration; untimed stages (null entries) are still launched
    w = WORKLOADS["tiny"].replace(T=128 * 16, Hqk=2, Hv=4, chunk=128, dtype="bf16", h0_std=0.05)
    x = make_inputs(w, device="cuda", seed=7 + ng)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    o1, h1 = gdn.chunk_fwd(*args, chunk=128, n_groups=ng)
    bits = [0, 3, 4] if ng <= 1 else [0, 1, 2, 3, 4]
    starts, stops = [None] * 5, [None] * 5
    for b in bits[:-1]:   # the last stage launched untimed
        for lst in (starts, stops):
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            lst[b] = e
    torch.cuda.synchronize()
    o2, h2 = gdn.chunk_fwd(*args, chunk=128, n_groups=ng, events=(starts, stops))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    for b in bits[:-1]:
        assert starts[b].elapsed_time(stops[b]) > 0


# ---------------------------------------------------------------------------
# rows a7-a9: fold, exclusive prefix, replay


@pytest.mark.parametrize("dtype,C", [("bf16", 128), ("f32", 64)])
def test_fold_matches_oracle(gdn, dtype, C):
    w = WORKLOADS["tiny"].replace(T=C * 8, Hqk=1, Hv=2, chunk=C, dtype=dtype)
    x = make_inputs(w, device="cuda", seed=11, g_const=-0.01)   # weak decay: A far from 0
    A, Bm = gdn.chunk_fold(x["k"], x["v"], x["g"], x["beta"], n_groups=4, chunk=C)
    torch.cuda.synchronize()
    Ar, Br = oracle.fold(_cpu(x["k"]), _cpu(x["v"]), _cpu(x["g"]), _cpu(x["beta"]), n_groups=4)
    # A decays towards zero with most entries tiny, so errors are scaled by
    # the largest entry.  bf16 path: the walk's W x state product takes bf16
    # operands (relative 2^-9 each) over 2 chunks per group -> 1e-2 of max.
    # fp32 path: fp32 products, 1e-4 of max.
    tol = 1e-2 if dtype == "bf16" else 1e-4
    assert _err(A.cpu().numpy(), Ar) <= tol * np.abs(Ar).max()
    assert _err(Bm.cpu().numpy(), Br) <= tol * np.abs(Br).max()


@pytest.mark.parametrize("dtype,C,Hqk,Hv,ng,cpj", [
    ("bf16", 128, 4, 8, 32, 2),    # 256 group-walks, 512 workgroup items: the persistent fold, halves alternating
    ("bf16", 128, 5, 10, 30, 2),   # 600 items (not whole blocks of the grid): persistent, halves not alternated
    ("bf16", 128, 4, 8, 32, 3),    # an odd chunk count per group: one workgroup per item
    ("bf16", 128, 2, 8, 32, 2),    # four value heads per qk head, placed side by side
    ("bf16", 64, 4, 8, 32, 2),
    ("f32", 64, 4, 8, 32, 2),
])
def test_fold_throughput_forms(gdn, dtype, C, Hqk, Hv, ng, cpj):
    # the fold of 256 or more group-walks (8 slices per workgroup, two
    # workgroups per group), against the oracle's fold of every group
    w = WORKLOADS["tiny"].replace(T=C * cpj * ng, Hqk=Hqk, Hv=Hv, chunk=C, dtype=dtype)
    x = make_inputs(w, device="cuda", seed=ng + cpj, g_const=-0.01)   # weak decay: A far from 0
    A, Bm = gdn.chunk_fold(x["k"], x["v"], x["g"], x["beta"], n_groups=ng, chunk=C)
    torch.cuda.synchronize()
    Ar, Br = oracle.fold(_cpu(x["k"]), _cpu(x["v"]), _cpu(x["g"]), _cpu(x["beta"]), n_groups=ng)
    # bars as in test_fold_matches_oracle (errors scaled by the largest entry)
    tol = 1e-2 if dtype == "bf16" else 1e-4
    assert _err(A.cpu().numpy(), Ar) <= tol * np.abs(Ar).max()
    assert _err(Bm.cpu().numpy(), Br) <= tol * np.abs(Br).max()


@pytest.mark.parametrize("split", [False, True])
def test_compose_prefix_matches_oracle(gdn, split):
    BH, n = 3, 9
    gen = torch.Generator().manual_seed(12)
    A = (torch.randn(BH, n, 128, 128, generator=gen) * (0.9 / 128 ** 0.5)).float()
    Bm = torch.randn(BH, n, 128, 128, generator=gen).float()
    h0 = torch.randn(BH, 128, 128, generator=gen).float()
    h_in, h_fin = gdn.compose_prefix(A.cuda(), Bm.cuda(), h0.cuda(), split_bf16=split)
    torch.cuda.synchronize()
    r_in, r_fin = oracle.prefix(A.numpy(), Bm.numpy(), h0.numpy())
    # fp32 products: 128-term dots at unit roundoff 6e-8 carried over 9
    # contracting steps stay within ~1e-5 of RMS; hi/lo bf16 splitting drops
    # terms of relative size 2^-16 -> 1e-4.
    tol = 1e-4 if split else 2e-5
    assert _err(h_in.cpu().numpy(), r_in) <= tol * _rms(r_in)
    assert _err(h_fin.cpu().numpy(), r_fin) <= tol * _rms(r_fin)


@pytest.mark.parametrize("n", [35, 37, 48, 64, 256])
@pytest.mark.parametrize("split", [False, True])
def test_blocked_prefix_matches_oracle(gdn, n, split):
    # Three rows of 35..256 pairs, the blocked prefix forced (each block of
    # ~sqrt(n) pairs composed, the prefix over the blocks, every block
    # replayed) -- blocks of 5 (n = 35), 6 (48), 8 (64) and 16 (256) pairs;
    # 37 pairs (prime) have no blocks and take the sequential prefix.
    # Against the oracle's one-pair-at-a-time prefix, and against the
    # library's sequential one (GDN_PREFIX_SEQUENTIAL)
    BH = 3
    gen = torch.Generator().manual_seed(100 + n)
    A = (torch.randn(BH, n, 128, 128, generator=gen) * (0.95 / 128 ** 0.5)).float()
    Bm = torch.randn(BH, n, 128, 128, generator=gen).float()
    h0 = torch.randn(BH, 128, 128, generator=gen).float()
    h_in, h_fin = gdn.compose_prefix(A.cuda(), Bm.cuda(), h0.cuda(), split_bf16=split, form="blocked")
    s_in, s_fin = gdn.compose_prefix(A.cuda(), Bm.cuda(), h0.cuda(), split_bf16=split, form="sequential")
    c_in, c_fin = gdn.compose_prefix(A.cuda(), Bm.cuda(), h0.cuda(), split_bf16=split)
    torch.cuda.synchronize()
    # the chosen form is one of the two, bit for bit
    assert torch.equal(c_in, h_in) or torch.equal(c_in, s_in)
    r_in, r_fin = oracle.prefix(A.numpy(), Bm.numpy(), h0.numpy())
    # fp32: as for nine pairs.  Split bf16: each step adds rounding of
    # relative size ~2^-16 (the dropped lo*lo terms); along a chain with
    # contraction 0.95 those add up to about sqrt(1 / (1 - 0.95^2)) ~ 3.2
    # times one step's, and the max runs over ~30x more elements than the
    # nine-pair case's 1e-4 -> 5e-4
    tol = 5e-4 if split else 2e-5
    for name, got, ref in (("h_in", h_in, r_in), ("h_final", h_fin, r_fin), ("h_in seq", s_in, r_in)):
        e = _err(got.cpu().numpy(), ref)
        print(f"  {name}: max-abs {e:.3e}  limit {tol * _rms(ref):.3e}", flush=True)
        assert e <= tol * _rms(ref)


@pytest.mark.parametrize("ng", [2, 4, 16])
def test_group_count_invariance(gdn, ng):
    w = WORKLOADS["qwen3next_8b_layer"].replace(T=2048)
    x = make_inputs(w, device="cuda", seed=13)
    o, h, o_ref, h_ref = _run_and_compare(gdn, w, x, n_groups=ng)
    ro = _rms(o_ref)
    _check("o", o, o_ref, 2e-2, ro)
    _check("h_T", h, h_ref, 2e-2, ro)


@pytest.mark.parametrize("ng", [64, 72])
def test_many_groups_of_one_chunk(gdn, ng):
    # one chunk per group: the fold, a 64- or 72-step prefix and the replay
    # carry the whole sequence; weak decay so that every group's pair
    # reaches the output
    w = WORKLOADS["tiny"].replace(T=64 * ng, Hqk=1, Hv=2, chunk=64, dtype="bf16", h0_std=0.05)
    x = make_inputs(w, device="cuda", seed=ng, g_const=-0.01, beta_scale=0.1)
    o, h, o_ref, h_ref = _run_and_compare(gdn, w, x, n_groups=ng)
    ro = _rms(o_ref)
    _check("o", o, o_ref, 2e-2, ro)
    _check("h_T", h, h_ref, 2e-2, ro)


def test_groups_weak_decay_compose_matters(gdn):
    # g = 0 and small beta keep each group's affine map far from zero, so the
    # incoming states really carry information across groups
    w = WORKLOADS["tiny"].replace(T=2048, Hqk=2, Hv=2, chunk=128, dtype="bf16", h0_std=0.02, B=1)
    x = make_inputs(w, device="cuda", seed=14, g_const=0.0, beta_scale=0.1)
    o, h, o_ref, h_ref = _run_and_compare(gdn, w, x, n_groups=8)
    ro = _rms(o_ref)
    _check("o", o, o_ref, 2e-2, ro)
    _check("h_T", h, h_ref, 2e-2, ro)
    # h_T as the prefix composes it (all eight pairs applied to h0) equals the
    # last group's replayed end state, which the full call returns
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    o_p = torch.empty((w.B, w.T, w.Hv, w.dv), dtype=torch.float32, device="cuda")
    h_p = torch.empty((w.B, w.Hv, w.dk, w.dv), dtype=torch.float32, device="cuda")
    gdn.chunk_fwd(*args, chunk=128, n_groups=8, out=o_p, final_state=h_p,
                  stages=gdn.STAGE_PREP | gdn.STAGE_FOLD | gdn.STAGE_PREFIX)
    torch.cuda.synchronize()
    _check("h_T (prefix)", h_p.cpu().numpy(), h_ref, 2e-2, ro)
    _check("h_T (prefix vs replay)", h_p.cpu().numpy(), h.astype(np.float64), 2e-2, ro)
    # negative control: groups replayed from a zero state miss by far
    L = 256
    bad = []
    for j in range(8):
        s = slice(j * L, (j + 1) * L)
        oj, _ = gdn.chunk_fwd(x["q"][:, s].contiguous(), x["k"][:, s].contiguous(),
                              x["v"][:, s].contiguous(), x["g"][:, s].contiguous(),
                              x["beta"][:, s].contiguous(), None, chunk=128)
        bad.append(oj)
    bad = torch.cat(bad, dim=1).float().cpu().numpy()
    assert _err(bad, o_ref) > 10 * 2e-2 * ro


@pytest.mark.parametrize("dtype,C,B,Hqk,Hv,T,gc", [
    ("bf16", 128, 1, 2, 4, 1000, -0.01),    # the latency form of the walk, weak decay, ragged
    ("bf16", 128, 4, 16, 32, 640, None),    # 128 walks: the walk with outputs
    ("bf16", 64, 8, 8, 16, 64 * 7, -0.01),  # C = 64, 128 walks, weak decay
    ("f32", 64, 2, 1, 3, 64 * 5 - 3, -0.01),
])
def test_forward_affine(gdn, dtype, C, B, Hqk, Hv, T, gc):
    # gdn_chunk_fwd_affine: the walk of [A | h] from [I | h0] also yields the
    # map A of the whole sequence.  o and h_T are gdn_chunk_fwd's, bit for
    # bit; A is the oracle's product of the per-token maps (its fold of the
    # sequence as one group), and h_T = A h0 + B with B the oracle's state
    # reached from zero.
    w = WORKLOADS["tiny"].replace(T=T, B=B, Hqk=Hqk, Hv=Hv, chunk=C, dtype=dtype, h0_std=0.05)
    x = make_inputs(w, device="cuda", seed=T + B * Hv, g_const=gc, beta_scale=0.3 if gc is not None else None)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    o, hT, A = gdn.chunk_fwd_affine(*args, chunk=C)
    o1, h1 = gdn.chunk_fwd(*args, chunk=C)
    torch.cuda.synchronize()
    assert torch.equal(o, o1) and torch.equal(hT, h1)
    Ar, Br = oracle.fold(_cpu(x["k"]), _cpu(x["v"]), _cpu(x["g"]), _cpu(x["beta"]), n_groups=1)
    Ar, Br = Ar[:, :, 0], Br[:, :, 0]
    # (A: W x state products take bf16 operands on the bf16 path)
    tol = 1e-2 if dtype == "bf16" else 1e-4
    ea = _err(A.cpu().numpy(), Ar)
    print(f"  A: max-abs {ea:.3e} (max |A| {np.abs(Ar).max():.3e})", flush=True)
    assert ea <= tol * np.abs(Ar).max()
    hr = np.einsum("bhij,bhjc->bhic", Ar, x["h0"].cpu().double().numpy()) + Br
    o_ref, h_ref = oracle.fwd(**{kk: _cpu(vv) for kk, vv in x.items()})
    assert np.abs(hr - h_ref).max() <= 1e-9 * max(1.0, np.abs(h_ref).max())   # (the oracle's own identity)
    ro = _rms(o_ref)
    _check("o", o.cpu().numpy(), o_ref, TOL[dtype], ro)
    _check("h_T", hT.cpu().numpy(), h_ref, TOL[dtype], ro)


@pytest.mark.parametrize("C", [64, 128])
def test_sequence_shards_through_the_boundary(gdn, C):
    # The sequence-sharded flow, each shard standing in for a device, through
    # the exported entry points only.  First pass: every shard runs the
    # forward from a zero state with its affine map (gdn_chunk_fwd_affine):
    # its pair is (A, h_T).  The pairs are gathered and their exclusive prefix
    # (gdn_compose_prefix) gives each shard its incoming state; the second
    # pass, each shard's forward from that state (gdn_chunk_fwd), gives its
    # outputs.  Together they are the whole sequence's o and h_T.  Weak decay
    # keeps each shard's map far from zero, so the incoming states carry the
    # earlier shards.
    S, L = 4, 4 * C
    w = WORKLOADS["tiny"].replace(T=S * L, Hqk=2, Hv=4, chunk=C, dtype="bf16", h0_std=0.05, B=2)
    x = make_inputs(w, device="cuda", seed=40 + C, g_const=0.0, beta_scale=0.1)
    shard = lambda t, d: t[:, d * L:(d + 1) * L].contiguous()
    A, Bm = [], []
    for d in range(S):
        _, b_, a_ = gdn.chunk_fwd_affine(*[shard(x[kk], d) for kk in ("q", "k", "v", "g", "beta")], None, chunk=C)
        A.append(a_)
        Bm.append(b_)
    BH = w.B * w.Hv
    A = torch.stack(A, dim=2).reshape(BH, S, 128, 128)
    Bm = torch.stack(Bm, dim=2).reshape(BH, S, 128, 128)
    h_in, h_fin = gdn.compose_prefix(A, Bm, x["h0"].reshape(BH, 128, 128), split_bf16=True)
    outs, h_last = [], None
    for d in range(S):
        o_d, h_last = gdn.chunk_fwd(*[shard(x[kk], d) for kk in ("q", "k", "v", "g", "beta")],
                                    h_in[:, d].reshape(w.B, w.Hv, 128, 128).contiguous(), chunk=C)
        outs.append(o_d)
    torch.cuda.synchronize()
    o = torch.cat(outs, dim=1).float().cpu().numpy()
    o_ref, h_ref = oracle.fwd(**{kk: _cpu(vv) for kk, vv in x.items()})
    ro = _rms(o_ref)
    _check("o", o, o_ref, 2e-2, ro)
    _check("h_T (last shard)", h_last.cpu().numpy(), h_ref, 2e-2, ro)
    _check("h_T (prefix)", h_fin.reshape(w.B, w.Hv, 128, 128).cpu().numpy(), h_ref, 2e-2, ro)
    # the first pass's pairs equal the exported fold's (one group per shard)
    for d in (0, S - 1):
        Af, Bf = gdn.chunk_fold(*[shard(x[kk], d) for kk in ("k", "v", "g", "beta")], n_groups=1, chunk=C)
        torch.cuda.synchronize()
        ra = float((A[:, d] - Af.reshape(BH, 128, 128)).abs().max()) / float(Af.abs().max())
        rb = float((Bm[:, d] - Bf.reshape(BH, 128, 128)).abs().max()) / float(Bf.abs().max())
        assert ra <= 1e-2 and rb <= 1e-2, (d, ra, rb)
    # negative control: shards started from zero states miss by far
    o0 = torch.cat([gdn.chunk_fwd(*[shard(x[kk], d) for kk in ("q", "k", "v", "g", "beta")], None, chunk=C)[0]
                    for d in range(S)], dim=1).float().cpu().numpy()
    assert _err(o0, o_ref) > 10 * 2e-2 * ro


@pytest.mark.parametrize("dtype,C,B,Hqk,Hv,T", [
    ("f32", 64, 1, 2, 2, 512),      # the tiny workload's shape
    ("bf16", 128, 1, 2, 4, 640),    # 8B-layer heads ratio, five chunks
    ("bf16", 64, 2, 1, 2, 64 * 4 - 21),   # partial last chunk
])
def test_bwd_state_matches_oracle(gdn, dtype, C, B, Hqk, Hv, T):
    # the backward's reverse chunk walk (gdn_chunk_bwd_state): the cotangent
    # of every chunk's incoming state and of h0, against the chunked fp64
    # gradient of the rule (oracle/backward.py: chunked_bwd, itself pinned by
    # finite differences and against the per-token reverse pass).  Bars as
    # for the forward, relative to the RMS of the oracle's cotangents.
    from oracle import backward

    w = WORKLOADS["tiny"].replace(T=T, B=B, Hqk=Hqk, Hv=Hv, chunk=C, dtype=dtype, h0_std=0.05)
    x = make_inputs(w, device="cuda", seed=T + Hv)
    gen = torch.Generator().manual_seed(T + 7)
    dO = torch.randn((B, T, Hv, 128), generator=gen).to("cuda")
    dhT = (torch.randn((B, Hv, 128, 128), generator=gen) * 0.1).to("cuda")
    dhc, dh0 = gdn.chunk_bwd_state(x["q"], x["k"], x["g"], x["beta"], dO, dhT, chunk=C)
    torch.cuda.synchronize()
    out, walk, _ = backward.chunked_bwd(*[_cpu(x[kk]) for kk in ("q", "k", "v", "g", "beta")], _cpu(x["h0"]),
                                        do=_cpu(dO), dhT=_cpu(dhT), C=C, return_walk=True)
    r = _rms(walk)
    for name, got, ref in (("dh_n", dhc.cpu().numpy(), walk), ("dh0", dh0.cpu().numpy(), out["dh0"])):
        e = _err(got, ref)
        print(f"  {name}: max-abs {e:.3e}  limit {TOL[dtype] * r:.3e}", flush=True)
        assert e <= TOL[dtype] * r
    # dh_T = 0 and dO = 0 give zero cotangents; dO = 0 alone gives the
    # transposed maps applied to dh_T only (ddh = 0)
    z = torch.zeros_like(dO)
    dhz, dh0z = gdn.chunk_bwd_state(x["q"], x["k"], x["g"], x["beta"], z, None, chunk=C)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dhz) == 0 and torch.count_nonzero(dh0z) == 0


@pytest.mark.parametrize("dtype,C,B,Hqk,Hv,T", [
    ("f32", 64, 1, 1, 2, 200),       # fp32, partial last chunk, two value heads per key head
    ("bf16", 128, 1, 2, 4, 300),     # chunk 128, partial last chunk
    ("bf16", 64, 2, 1, 1, 128),      # whole chunks, two batch rows
    ("bf16", 64, 1, 2, 2, 50),       # shorter than one chunk
])
def test_bwd_grads_match_oracle(gdn, dtype, C, B, Hqk, Hv, T):
    # the full backward (gdn_chunk_bwd): dq, dk, dv, dg, dbeta, dh0 against
    # the oracle's per-token reverse pass of the rule (oracle/backward.py:
    # bwd, pinned by finite differences), with a non-zero h0 and dh_T.  Bars
    # relative to the RMS of each oracle gradient: fp32 as for the forward;
    # bf16 inputs 1e-3 -- unlike the forward's bf16 W x h products, every
    # product of the backward takes its fp32 operands as hi/lo bf16 halves
    # (about 2^-16 relative each), chained through about ten products and
    # the two walks
    from oracle import backward
    tol = {"f32": 1e-4, "bf16": 1e-3}[dtype]

    w = WORKLOADS["tiny"].replace(T=T, B=B, Hqk=Hqk, Hv=Hv, chunk=C, dtype=dtype, h0_std=0.05)
    x = make_inputs(w, device="cuda", seed=T + 3 * Hv + B)
    gen = torch.Generator().manual_seed(T + 11)
    dO = torch.randn((B, T, Hv, 128), generator=gen).to("cuda")
    dhT = (torch.randn((B, Hv, 128, 128), generator=gen) * 0.1).to("cuda")
    got = gdn.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], dO, h0=x["h0"], dh_T=dhT, chunk=C)
    torch.cuda.synchronize()
    ref = backward.bwd(*[_cpu(x[kk]) for kk in ("q", "k", "v", "g", "beta", "h0")], do=_cpu(dO), dhT=_cpu(dhT))
    for name in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        r = ref[name]
        e = _err(got[name].cpu().numpy(), r)
        print(f"  {name}: max-abs {e:.3e}  limit {tol * _rms(r):.3e}", flush=True)
        assert e <= tol * _rms(r), name
    # no cotangents: every gradient zero
    z = gdn.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], torch.zeros_like(dO), h0=x["h0"], chunk=C)
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        assert torch.count_nonzero(z[name]) == 0, name


@pytest.mark.timeout(900)
def test_bwd_grads_full_size(gdn):
    # the backward at the 4096-token layer's full size and in the launch
    # configuration the bench times (chunk 128, 16 key / 32 value heads, h0
    # drawn), every gradient element against the oracle's per-token reverse
    # pass of the rule (about ten seconds of host work); bar as for the small
    # cases
    from oracle import backward

    w = WORKLOADS["qwen3next_8b_layer"]
    x = make_inputs(w, device="cuda")
    gen = torch.Generator().manual_seed(77)
    dO = torch.randn((w.B, w.T, w.Hv, 128), generator=gen).to("cuda")
    dhT = (torch.randn((w.B, w.Hv, 128, 128), generator=gen) * 0.1).to("cuda")
    got = gdn.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], dO, h0=x["h0"], dh_T=dhT, chunk=w.chunk)
    torch.cuda.synchronize()
    got = {kk: vv.cpu().numpy() for kk, vv in got.items()}
    ref = backward.bwd(*[_cpu(x[kk]) for kk in ("q", "k", "v", "g", "beta", "h0")], do=_cpu(dO), dhT=_cpu(dhT))
    for name in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        r = ref[name]
        e = _err(got[name], r)
        print(f"  {name}: max-abs {e:.3e}  limit {1e-3 * _rms(r):.3e}", flush=True)
        assert e <= 1e-3 * _rms(r), name


@pytest.mark.parametrize("B,Hqk,Hv", [(1, 16, 32), (4, 8, 16)])
def test_bwd_workspace_reuse(gdn, B, Hqk, Hv):
    # one workspace (filled with 0xFF bytes first) for several backward calls
    # in a row on different inputs: no call may depend on what an earlier one
    # left in it.  Each call equals a call on a fresh workspace (to 1e-5 of
    # each gradient's RMS: the row sums gather through LDS atomics, whose
    # order is not fixed).
    w = WORKLOADS["qwen3next_8b_layer"].replace(T=1024 + 77, B=B, Hqk=Hqk, Hv=Hv)
    shape = gdn.make_shape(w.B, w.T, w.Hqk, w.Hv, 128, 128, 128, 0, torch.bfloat16, torch.float32)
    ws = torch.empty(gdn.workspace_size_bwd_grads(shape), dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)
    for seed in (11, 12, 13):
        x = make_inputs(w, device="cuda", seed=seed)
        gen = torch.Generator().manual_seed(seed)
        dO = torch.randn((w.B, w.T, w.Hv, 128), generator=gen).to("cuda")
        dhT = (torch.randn((w.B, w.Hv, 128, 128), generator=gen) * 0.1).to("cuda")
        args = (x["q"], x["k"], x["v"], x["g"], x["beta"], dO)
        got = gdn.chunk_bwd(*args, h0=x["h0"], dh_T=dhT, chunk=128, workspace=ws)
        ref = gdn.chunk_bwd(*args, h0=x["h0"], dh_T=dhT, chunk=128)
        torch.cuda.synchronize()
        for name in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
            r = ref[name].double()
            e = float((got[name].double() - r).abs().max())
            assert e <= 1e-5 * float(r.pow(2).mean().sqrt()), (seed, name, e)


def test_long_sequence_reduced(gdn):
    # the long-sequence workload's shape and group structure at 1/16 of its length
    w = WORKLOADS["long_256k"].replace(T=16384, n_groups=16)
    x = make_inputs(w, device="cuda")
    o, h, o_ref, h_ref = _run_and_compare(gdn, w, x)
    ro = _rms(o_ref)
    _check("o", o, o_ref, 2e-2, ro)
    _check("h_T", h, h_ref, 2e-2, ro)


@pytest.mark.parametrize("dtype,C,T,Hqk,Hv,h0,ng", [
    ("f32", 64, 64 * 5 + 17, 1, 3, 0.3, 0),       # fp32, partial last chunk
    ("bf16", 128, 128 * 9 + 1, 2, 4, 0.1, 0),     # a one-token last chunk
    ("bf16", 64, 63, 1, 2, 0.05, 0),              # shorter than one chunk
    ("bf16", 128, 4000, 2, 4, 0.02, 4),           # chunk-groups, the last one ragged
    ("bf16", 128, 4000, 8, 16, 0.02, 4),          # the same replayed by the walk with outputs (128 walks)
    ("bf16", 128, 4000, 8, 32, 0.02, 4),          # 256 replay walks: two state slices per wave, ragged
    ("bf16", 64, 64 * 9 + 5, 8, 16, 0.05, 5),     # C = 64, walk with outputs (160 walks), ragged
])
def test_forward_ragged_tail(gdn, dtype, C, T, Hqk, Hv, h0, ng):
    # T not a multiple of the chunk: the last chunk is padded with identity
    # steps inside the library; o and h_T must be those of the unpadded rule
    w = WORKLOADS["tiny"].replace(T=T, Hqk=Hqk, Hv=Hv, chunk=C, dtype=dtype, h0_std=h0, B=2)
    x = make_inputs(w, device="cuda", seed=T + C)
    o, h, o_ref, h_ref = _run_and_compare(gdn, w, x, n_groups=ng)
    ro = _rms(o_ref)
    _check("o", o, o_ref, TOL[dtype], ro)
    _check("h_T", h, h_ref, TOL[dtype], ro)


def _packed(gdn, dtype, C, lens, Hqk, Hv, h0_std, seed):
    # one packed row of the given sequence lengths, with per-sequence h0
    T = int(sum(lens))
    w = WORKLOADS["tiny"].replace(T=max(T, 1), Hqk=Hqk, Hv=Hv, chunk=C, dtype=dtype, h0_std=0.0, B=1)
    x = make_inputs(w, device="cuda", seed=seed)
    x = {kk: (vv[:, :T].contiguous() if vv is not None and kk != "h0" else vv) for kk, vv in x.items()}
    gen = torch.Generator().manual_seed(seed + 1)
    h0 = (torch.randn((len(lens), Hv, 128, 128), generator=gen) * h0_std).to("cuda")
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device="cuda")
    return x, h0, cu


@pytest.mark.parametrize("dtype,C", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_varlen_equals_separate_calls(gdn, dtype, C):
    # packed sequences (gdn_chunk_fwd_varlen) equal one gdn_chunk_fwd call per
    # sequence, bit for bit (same kernels, same arithmetic), including empty
    # and one-token sequences; and each matches the oracle
    lens = [0, 1, C - 1, C, C + 1, 3 * C + 7, 0, 2 * C]
    x, h0, cu = _packed(gdn, dtype, C, lens, 2, 4, 0.05, seed=C + len(dtype))
    o, hT = gdn.chunk_fwd_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], cu, h0, chunk=C)
    torch.cuda.synchronize()
    a = 0
    for s_, n in enumerate(lens):
        if n == 0:
            assert torch.equal(hT[s_], h0[s_])
            continue
        sl = slice(a, a + n)
        args = [x[kk][:, sl].contiguous() for kk in ("q", "k", "v", "g", "beta")]
        o1, h1 = gdn.chunk_fwd(*args, h0[s_:s_ + 1].contiguous(), chunk=C)
        torch.cuda.synchronize()
        assert torch.equal(o[:, sl], o1) and torch.equal(hT[s_:s_ + 1], h1), f"sequence {s_} (length {n})"
        o_ref, h_ref = oracle.fwd(*[t.cpu() for t in args], h0[s_:s_ + 1].cpu())
        ro = _rms(o_ref)
        _check(f"o[{s_}]", o1.float().cpu().numpy(), o_ref, TOL[dtype], ro)
        _check(f"h_T[{s_}]", h1.cpu().numpy(), h_ref, TOL[dtype], ro)
        a += n


def test_varlen_throughput_form(gdn):
    # 16 sequences x 32 value heads = 512 walks: the throughput form of the
    # walk and the separate output stage, against the oracle per sequence
    rng = np.random.default_rng(5)
    lens = [int(n) for n in rng.integers(1, 400, size=16)]
    x, h0, cu = _packed(gdn, "bf16", 128, lens, 16, 32, 0.02, seed=17)
    o, hT = gdn.chunk_fwd_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], cu, h0, chunk=128)
    torch.cuda.synchronize()
    a = 0
    for s_, n in enumerate(lens):
        sl = slice(a, a + n)
        o_ref, h_ref = oracle.fwd(*[x[kk][:, sl].cpu() for kk in ("q", "k", "v", "g", "beta")], h0[s_:s_ + 1].cpu())
        ro = _rms(o_ref)
        _check(f"o[{s_}]", o[:, sl].float().cpu().numpy(), o_ref, 2e-2, ro)
        _check(f"h_T[{s_}]", hT[s_:s_ + 1].cpu().numpy(), h_ref, 2e-2, ro)
        a += n


def test_varlen_many_short_sequences(gdn):
    # 2100 sequences of 1..20 tokens x 32 value heads (67,200 walks, more
    # than a padded batch allows): a sample of sequences against the oracle
    rng = np.random.default_rng(9)
    lens = [int(n) for n in rng.integers(1, 21, size=2100)]
    x, h0, cu = _packed(gdn, "bf16", 128, lens, 16, 32, 0.02, seed=23)
    o, hT = gdn.chunk_fwd_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], cu, h0, chunk=128)
    torch.cuda.synchronize()
    starts = np.concatenate([[0], np.cumsum(lens)])
    for s_ in list(range(0, 2100, 97)) + [2099]:
        sl = slice(int(starts[s_]), int(starts[s_ + 1]))
        o_ref, h_ref = oracle.fwd(*[x[kk][:, sl].cpu() for kk in ("q", "k", "v", "g", "beta")],
                                  h0[s_:s_ + 1].cpu())
        ro = _rms(o_ref)
        _check(f"o[{s_}]", o[:, sl].float().cpu().numpy(), o_ref, 2e-2, ro)
        _check(f"h_T[{s_}]", hT[s_:s_ + 1].cpu().numpy(), h_ref, 2e-2, ro)


def test_varlen_throughput_form_with_empty_sequences(gdn):
    # 24 sequences x 4 value heads = 96 walks (the 4-slice throughput form),
    # a third of them empty: those return h0 as h_T untouched, the others
    # match the oracle per sequence
    lens = [0 if i % 3 == 1 else 1 + (37 * i) % 300 for i in range(24)]
    x, h0, cu = _packed(gdn, "bf16", 128, lens, 2, 4, 0.05, seed=29)
    o, hT = gdn.chunk_fwd_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], cu, h0, chunk=128)
    torch.cuda.synchronize()
    a = 0
    for s_, n in enumerate(lens):
        if n == 0:
            assert torch.equal(hT[s_], h0[s_])
            continue
        sl = slice(a, a + n)
        if s_ % 4 == 0:   # a sample against the oracle
            o_ref, h_ref = oracle.fwd(*[x[kk][:, sl].cpu() for kk in ("q", "k", "v", "g", "beta")],
                                      h0[s_:s_ + 1].cpu())
            ro = _rms(o_ref)
            _check(f"o[{s_}]", o[:, sl].float().cpu().numpy(), o_ref, 2e-2, ro)
            _check(f"h_T[{s_}]", hT[s_:s_ + 1].cpu().numpy(), h_ref, 2e-2, ro)
        a += n


def test_varlen_bf16_output(gdn):
    # packed sequences with a bf16 o: the fp32-o call's values rounded once
    # (the output stage rounds its fp32 result), bit for bit
    lens = [70, 1, 300, 128]
    x, h0, cu = _packed(gdn, "bf16", 128, lens, 2, 4, 0.05, seed=31)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], cu, h0)
    o32, h32 = gdn.chunk_fwd_varlen(*args, chunk=128)
    o16, h16 = gdn.chunk_fwd_varlen(*args, chunk=128, o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o16, o32.to(torch.bfloat16)) and torch.equal(h16, h32)


def test_varlen_all_empty(gdn):
    # every sequence empty: h_T = h0 (and nothing else is touched)
    x, h0, cu = _packed(gdn, "bf16", 128, [0, 0, 0], 1, 2, 0.1, seed=3)
    q = torch.zeros((1, 0, 1, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((1, 0, 2, 128), dtype=torch.bfloat16, device="cuda")
    gb = torch.zeros((1, 0, 2), dtype=torch.float32, device="cuda")
    o, hT = gdn.chunk_fwd_varlen(q, q, v, gb, gb, cu, h0, chunk=128)
    o2, hT2 = gdn.chunk_fwd_varlen(q, q, v, gb, gb, [0, 0, 0, 0], h0, chunk=128)   # offsets as a list
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(hT, h0) and torch.equal(hT2, h0)


@pytest.mark.parametrize("C", [64, 128])
def test_forward_throughput_form(gdn, C):
    # 512 walks (B * H_v): the single walk takes its throughput form (eight
    # slices per workgroup sharing W and K^T through LDS) instead of the
    # latency form the shorter walks above take
    w = WORKLOADS["tiny"].replace(T=3 * C - 5, Hqk=16, Hv=32, chunk=C, dtype="bf16", h0_std=0.02, B=16)
    x = make_inputs(w, device="cuda", seed=C + 3)   # (with a partial last chunk)
    o, h, o_ref, h_ref = _run_and_compare(gdn, w, x)
    ro = _rms(o_ref)
    _check("o", o, o_ref, 2e-2, ro)
    _check("h_T", h, h_ref, 2e-2, ro)


@pytest.mark.parametrize("dtype,C,T,B,Hqk,Hv,h0", [
    ("bf16", 128, 2 * 128 + 1, 1, 3, 33, 0.02),   # 33 walks, 3 chunks (the last one token)
    ("bf16", 64, 5 * 64 - 3, 3, 4, 16, 0.0),      # 48 walks, partial last chunk
    ("f32", 64, 7 * 64, 2, 4, 20, 0.5),           # 40 walks, odd chunk count, strong h0
    ("bf16", 128, 4 * 128, 2, 32, 32, 0.1),       # 64 walks, as the dense layer
])
def test_forward_paired_form(gdn, dtype, C, T, B, Hqk, Hv, h0):
    # 33..64 walks (B * H_v): two slices of a head per workgroup sharing one
    # LDS copy of each chunk's W and K^T
    w = WORKLOADS["tiny"].replace(T=T, B=B, Hqk=Hqk, Hv=Hv, chunk=C, dtype=dtype, h0_std=h0)
    x = make_inputs(w, device="cuda", seed=T + B * Hv)
    o, h, o_ref, h_ref = _run_and_compare(gdn, w, x)
    ro = _rms(o_ref)
    _check("o", o, o_ref, TOL[dtype], ro)
    _check("h_T", h, h_ref, TOL[dtype], ro)


@pytest.mark.parametrize("dtype,C,T,B,Hqk,Hv", [
    ("bf16", 128, 3 * 128 - 7, 5, 13, 13),   # 65 walks: the 4-slice throughput form
    ("bf16", 128, 3 * 128 - 7, 3, 16, 32),   # 96 walks
    ("bf16", 64, 4 * 64 + 3, 4, 8, 24),      # 96 walks at C = 64, partial last chunk
    ("f32", 64, 3 * 64, 5, 4, 20),           # 100 walks, fp32
])
def test_forward_walk_form_thresholds(gdn, dtype, C, T, B, Hqk, Hv):
    # either side of the walk count at which the walk changes launch form
    w = WORKLOADS["tiny"].replace(T=T, B=B, Hqk=Hqk, Hv=Hv, chunk=C, dtype=dtype, h0_std=0.05)
    x = make_inputs(w, device="cuda", seed=B * Hv + C)
    o, h, o_ref, h_ref = _run_and_compare(gdn, w, x)
    ro = _rms(o_ref)
    _check("o", o, o_ref, TOL[dtype], ro)
    _check("h_T", h, h_ref, TOL[dtype], ro)


def test_varlen_paired_form(gdn):
    # 3 sequences x 16 value heads = 48 walks (the paired form), one of them
    # empty and one a single token, against the oracle per sequence
    lens = [0, 1, 3 * 128 + 50]
    x, h0, cu = _packed(gdn, "bf16", 128, lens, 4, 16, 0.05, seed=23)
    o, hT = gdn.chunk_fwd_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], cu, h0, chunk=128)
    torch.cuda.synchronize()
    assert torch.equal(hT[0], h0[0])
    a = 0
    for s_, n in enumerate(lens):
        if n == 0:
            continue
        sl = slice(a, a + n)
        o_ref, h_ref = oracle.fwd(*[x[kk][:, sl].cpu() for kk in ("q", "k", "v", "g", "beta")], h0[s_:s_ + 1].cpu())
        ro = _rms(o_ref)
        _check(f"o[{s_}]", o[:, sl].float().cpu().numpy(), o_ref, 2e-2, ro)
        _check(f"h_T[{s_}]", hT[s_:s_ + 1].cpu().numpy(), h_ref, 2e-2, ro)
        a += n


def _graph_replays_equal(fn, outs, refs, n=3):
    # capture fn (which writes into the tensors `outs`) in a HIP graph after
    # one warm-up call on a side stream, then replay it n times with eager
    # work (the outputs cleared by a fill kernel) and synchronisations in
    # between; every replay must give `refs` bit for bit
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    for r in range(n):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, ref in zip(outs, refs):
            assert torch.equal(t, ref), f"replay {r}"


@pytest.mark.parametrize("ng", [0, 4])
def test_graph_replay_equals_eager(gdn, ng):
    # the forward recorded in a HIP graph (no allocation, copy or memset inside
    # the library) and replayed gives the eager call's outputs, bit for bit
    w = WORKLOADS["qwen3next_8b_layer"].replace(T=2048)
    x = make_inputs(w, device="cuda", seed=51)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    o_ref, h_ref = gdn.chunk_fwd(*args, chunk=128, n_groups=ng)
    shape = gdn.make_shape(w.B, w.T, w.Hqk, w.Hv, 128, 128, 128, ng, x["k"].dtype, torch.float32)
    ws = torch.empty(gdn.workspace_size(shape), dtype=torch.uint8, device="cuda")
    o, hT = torch.empty_like(o_ref), torch.empty_like(h_ref)
    _graph_replays_equal(lambda: gdn.chunk_fwd(*args, chunk=128, n_groups=ng, workspace=ws, out=o, final_state=hT),
                         (o, hT), (o_ref, h_ref))


def test_graph_replay_equals_eager_packed(gdn):
    # packed sequences: the chunk tables are built on the device inside the graph
    lens = [5, 300, 0, 129, 1000]
    x, h0, cu = _packed(gdn, "bf16", 128, lens, 2, 4, 0.05, seed=52)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], cu, h0)
    o_ref, h_ref = gdn.chunk_fwd_varlen(*args, chunk=128)
    shape = gdn.make_shape(len(lens), sum(lens), 2, 4, 128, 128, 128, 0, torch.bfloat16, torch.float32)
    ws = torch.empty(gdn.workspace_size_varlen(shape), dtype=torch.uint8, device="cuda")
    o, hT = torch.empty_like(o_ref), torch.empty_like(h_ref)
    _graph_replays_equal(lambda: gdn.chunk_fwd_varlen(*args, chunk=128, workspace=ws, out=o, final_state=hT),
                         (o, hT), (o_ref, h_ref))


class _Stream:
    """Running max-abs error and sum of squares of a reference, block by block."""

    def __init__(self):
        self.err, self.ss, self.n = 0.0, 0.0, 0

    def add(self, got, ref):
        self.err = max(self.err, _err(got, ref))
        self.ss += float(np.sum(np.square(ref, dtype=np.float64)))
        self.n += ref.size

    @property
    def rms(self):
        return (self.ss / max(self.n, 1)) ** 0.5


@pytest.mark.timeout(1500)
@pytest.mark.parametrize("name", ["long_256k", "million_1m"])
def test_long_sequence_full_size(gdn, name):
    # Full length, in the benchmark's launch configuration (256 chunk-groups:
    # fold, exclusive prefix, replay), every value head and state column
    # against the oracle, streamed over blocks of heads.  The grouped result
    # must also match one sequential walk over all chunks (the composition
    # checked against a sequential single-device reference: "GatedDeltaNet
    # does not support ici_context_parallelism", section "Status"), and the
    # prefix's composition of all pairs must equal the last group's replayed
    # end state.
    w = WORKLOADS[name]
    x = make_inputs(w, device="cuda")
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    o_g, h_g = gdn.chunk_fwd(*args, chunk=w.chunk, n_groups=w.n_groups)
    # the prefix's final state: the same call without the replay and output
    h_p = torch.empty_like(h_g)
    gdn.chunk_fwd(*args, chunk=w.chunk, n_groups=w.n_groups, out=o_g, final_state=h_p,
                  stages=gdn.STAGE_PREP | gdn.STAGE_FOLD | gdn.STAGE_PREFIX)
    torch.cuda.synchronize()
    h_g_np, h_p_np = h_g.cpu().numpy(), h_p.cpu().numpy()
    o_s, h_s = gdn.chunk_fwd(*args, chunk=w.chunk, n_groups=0)
    torch.cuda.synchronize()
    h_s_np = h_s.cpu().numpy()
    xc = {kk: _cpu(vv) for kk, vv in x.items()}
    del x, args
    torch.cuda.empty_cache()
    rep = w.Hv // w.Hqk
    blk = 4 if w.T <= 262144 else 2          # value heads per oracle block
    st = {k_: _Stream() for k_ in ("o_g", "o_s", "o_gs", "h_g", "h_s", "h_gs", "h_p")}
    for h0_ in range(0, w.Hv, blk):
        h1_ = h0_ + blk
        q0, q1 = h0_ // rep, (h1_ - 1) // rep + 1
        sub = dict(q=xc["q"][:, :, q0:q1].contiguous(), k=xc["k"][:, :, q0:q1].contiguous(),
                   v=xc["v"][:, :, q0 * rep:q1 * rep].contiguous(),
                   g=xc["g"][:, :, q0 * rep:q1 * rep].contiguous(),
                   beta=xc["beta"][:, :, q0 * rep:q1 * rep].contiguous(),
                   h0=xc["h0"][:, q0 * rep:q1 * rep].contiguous() if xc["h0"] is not None else None)
        o_ref, h_ref = oracle.fwd(**sub, heads=(h0_ - q0 * rep, h1_ - q0 * rep))
        og = o_g[:, :, h0_:h1_].cpu().numpy()
        os_ = o_s[:, :, h0_:h1_].cpu().numpy()
        st["o_g"].add(og, o_ref)
        st["o_s"].add(os_, o_ref)
        st["o_gs"].add(og, os_.astype(np.float64))
        del og, os_, o_ref
        st["h_g"].add(h_g_np[:, h0_:h1_], h_ref)
        st["h_s"].add(h_s_np[:, h0_:h1_], h_ref)
        st["h_p"].add(h_p_np[:, h0_:h1_], h_ref)
        st["h_gs"].add(h_g_np[:, h0_:h1_], h_s_np[:, h0_:h1_].astype(np.float64))
        print(f"  heads {h0_}..{h1_ - 1}: o grouped {st['o_g'].err:.3e}, single {st['o_s'].err:.3e}",
              flush=True)
    ro, rh = st["o_g"].rms, st["h_g"].rms
    tol = TOL[w.dtype]
    for k_, r in (("o_g", ro), ("o_s", ro), ("o_gs", ro), ("h_g", min(rh, ro)), ("h_s", min(rh, ro)),
                  ("h_p", min(rh, ro)), ("h_gs", min(rh, ro))):
        print(f"  {k_}: max-abs {st[k_].err:.3e}  limit {tol * r:.3e}", flush=True)
        assert st[k_].err <= tol * r, f"{k_}: {st[k_].err:.3e} > {tol * r:.3e}"
    # the prefix's composition and the last group's replay: the same state
    d = float(np.abs(h_p_np - h_g_np).max())
    print(f"  prefix h_T vs replayed h_T: {d:.3e}", flush=True)
    assert d <= tol * min(rh, ro)
