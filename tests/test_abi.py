"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def gdn():
    import linear_attention_rnn_gdn_amd as g

    if not os.path.exists(g.LIB_PATH):
        from linear_attention_rnn_gdn_amd import build

        build.build()
    g.lib()
    return g


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "gdn.h")).read()
    return sorted(set(re.findall(r"^(?:gdn_status|size_t|const char \*)\s*(gdn_\w+)\(", text, re.M)))


def test_header_declares_expected_entry_points():
    syms = _declared_symbols()
    for s in ("gdn_chunk_fwd", "gdn_compose_prefix", "gdn_chunk_fold", "gdn_chunk_transform",
              "gdn_workspace_size", "gdn_validate", "gdn_status_str"):
        assert s in syms


def test_library_exports_every_declared_symbol(gdn):
    L = ctypes.CDLL(gdn.LIB_PATH)
    for s in _declared_symbols():
        assert hasattr(L, s), s
    assert set(_declared_symbols()) <= set(gdn.SYMBOLS) | {"gdn_status_str"}


def test_status_strings(gdn):
    L = gdn.lib()
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert L.gdn_status_str(code)
    assert L.gdn_status_str(0) == b"ok"


def _shape(gdn, **kw):
    import torch

    d = dict(B=1, T=4096, H_qk=16, H_v=32, d_k=128, d_v=128, chunk=128, n_groups=0,
             dtype=torch.bfloat16, o_dtype=torch.float32)
    d.update(kw)
    return gdn.make_shape(**d)


@pytest.mark.parametrize("kw,status", [
    ({}, 0),
    (dict(chunk=64), 0),
    (dict(T=0), 0),
    (dict(n_groups=4), 0),
    (dict(n_groups=32), 0),
    (dict(n_groups=3), -2),            # does not divide the 32 chunks
    (dict(n_groups=-1), -2),
    (dict(T=4100), 0),                 # ragged tail: the last chunk padded with identity steps
    (dict(T=4100, n_groups=33), 0),    # 33 chunks
    (dict(T=4100, n_groups=32), -2),   # does not divide the 33 chunks
    (dict(chunk=96), -2),
    (dict(d_k=64), -2),
    (dict(d_v=256), -2),
    (dict(H_v=24), -2),                # not a multiple of H_qk
    (dict(B=0), -2),
    (dict(T=-128), -2),
    (dict(T=128 * 70000), -2),         # more chunks than one grid dimension holds
])
def test_validate(gdn, kw, status):
    assert gdn.validate(_shape(gdn, **kw)) == status


def test_validate_dtypes(gdn):
    s = _shape(gdn)
    s.dtype = 7
    assert gdn.validate(s) == -3
    s = _shape(gdn)
    s.o_dtype = 2
    assert gdn.validate(s) == -3
    import torch

    # fp32 inputs are supported at chunk 64 only
    assert gdn.validate(_shape(gdn, dtype=torch.float32, chunk=64)) == 0
    assert gdn.validate(_shape(gdn, dtype=torch.float32, chunk=128)) == -2


def test_workspace_size_scales(gdn):
    a = gdn.workspace_size(_shape(gdn))
    b = gdn.workspace_size(_shape(gdn, T=8192))
    assert a > 0 and b > a
    # with 128 walks or more the walk forms the outputs itself and the
    # workspace holds no chunk-start states or corrected values: the grouped
    # problem (256 walks) needs only the pairs and incoming states more than
    # the same batch of 128 walks, which needs less than twice 32 walks
    d = gdn.workspace_size(_shape(gdn, B=4))
    c = gdn.workspace_size(_shape(gdn, B=4, n_groups=2))
    assert c > d and d < 2 * a
    with pytest.raises(gdn.GdnError):
        gdn.workspace_size(_shape(gdn, chunk=96))


def _fake(addr):
    return ctypes.c_void_p(addr)


def test_entry_points_reject_bad_arguments_without_launching(gdn):
    L = gdn.lib()
    s = _shape(gdn)
    ws = gdn.workspace_size(s)
    ok = _fake(1 << 20)
    odd = _fake((1 << 20) + 4)
    P = lambda *a: [x for x in a]
    null = None
    # NULL input
    assert L.gdn_chunk_fwd(ctypes.byref(s), null, ok, ok, ok, ok, null, ok, null, ok, ws, null) == -1
    # misaligned
    assert L.gdn_chunk_fwd(ctypes.byref(s), odd, ok, ok, ok, ok, null, ok, null, ok, ws, null) == -4
    # workspace too small
    assert L.gdn_chunk_fwd(ctypes.byref(s), ok, ok, ok, ok, ok, null, ok, null, ok, ws - 1, null) == -5
    # bad shape
    bad = _shape(gdn, chunk=96)
    assert L.gdn_chunk_fwd(ctypes.byref(bad), ok, ok, ok, ok, ok, null, ok, null, ok, ws, null) == -2
    # fold / transform / prefix
    assert L.gdn_chunk_fold(ctypes.byref(s), ok, ok, ok, ok, null, ok, ok, ws, null) == -1
    assert L.gdn_chunk_transform(ctypes.byref(s), ok, ok, ok, ok, null, null, ok, ok, null) == -1
    assert L.gdn_compose_prefix(4, 8, 128, 128, ok, ok, null, null, null, 0, null) == -1
    assert L.gdn_compose_prefix(4, 8, 64, 128, ok, ok, null, ok, null, 0, null) == -2
    assert L.gdn_compose_prefix(0, 8, 128, 128, ok, ok, null, ok, null, 0, null) == -2
    assert L.gdn_compose_prefix(4, 8, 128, 128, odd, ok, null, ok, null, 0, null) == -4
    # sequential and blocked forced together
    assert L.gdn_compose_prefix(4, 8, 128, 128, ok, ok, null, ok, null, 6, null) == -2
    assert L.gdn_validate(None) == -1
    # the forward with the affine map: one group only, A required
    assert L.gdn_chunk_fwd_affine(ctypes.byref(s), ok, ok, ok, ok, ok, null, ok, null, null, ok, ws, null) == -1
    assert L.gdn_chunk_fwd_affine(ctypes.byref(s), ok, ok, ok, ok, ok, null, ok, null, odd, ok, ws, null) == -4
    grouped = _shape(gdn, n_groups=4)
    assert L.gdn_chunk_fwd_affine(ctypes.byref(grouped), ok, ok, ok, ok, ok, null, ok, null, ok, ok, ws, null) == -2


def test_backward_checks_without_launching(gdn):
    # gdn_chunk_bwd and gdn_chunk_bwd_state: one walk per sequence (no
    # chunk-groups), every input and gradient required (dh0 optional), 16-byte
    # alignment, workspace size; all rejected before anything is launched
    L = gdn.lib()
    s = _shape(gdn)
    ws = gdn.workspace_size_bwd_grads(s)
    assert ws > gdn.workspace_size(s)
    assert gdn.workspace_size_bwd_grads(_shape(gdn, T=8192)) > ws
    with pytest.raises(gdn.GdnError):
        gdn.workspace_size_bwd_grads(_shape(gdn, n_groups=4))
    ok = _fake(1 << 20)
    odd = _fake((1 << 20) + 4)
    null = None
    good = [ok] * 8 + [ok] * 5 + [null]   # q k v g beta h0 dO dh_T | dq dk dv dg dbeta | dh0
    def call(args, shape=s, nbytes=ws):
        return L.gdn_chunk_bwd(ctypes.byref(shape), *args, ok, nbytes, null)
    for i in (0, 1, 2, 3, 4, 6, 8, 9, 10, 11, 12):   # required pointers
        args = list(good)
        args[i] = null
        assert call(args) == -1, i
    for i in range(14):
        args = list(good)
        args[i] = odd
        assert call(args) == -4, i
    assert call(good, nbytes=ws - 1) == -5
    assert call(good, shape=_shape(gdn, n_groups=4)) == -2
    assert call(good, shape=_shape(gdn, chunk=96)) == -2
    # the state cotangents alone: at least one output
    assert L.gdn_chunk_bwd_state(ctypes.byref(s), ok, ok, ok, ok, ok, null, null, null, ok, ws, null) == -1


def test_varlen_checks_without_launching(gdn):
    # packed sequences: one walk per sequence (no chunk-groups); NULL offsets
    # are rejected before anything is launched
    L = gdn.lib()
    s = _shape(gdn, B=8, T=1000)
    ws = gdn.workspace_size_varlen(s)
    assert ws > 0
    assert gdn.workspace_size_varlen(_shape(gdn, B=8, T=1000, n_groups=1)) == ws
    with pytest.raises(gdn.GdnError):
        gdn.workspace_size_varlen(_shape(gdn, B=8, T=1000, n_groups=4))
    ok = _fake(1 << 20)
    null = None
    assert L.gdn_chunk_fwd_varlen(ctypes.byref(s), null, ok, ok, ok, ok, ok, null, ok, null, ok, ws, null) == -1
    assert L.gdn_chunk_fwd_varlen(ctypes.byref(s), ok, ok, ok, ok, ok, ok, null, ok, null, ok, ws - 1, null) == -5
    assert L.gdn_chunk_fwd_varlen(ctypes.byref(s), _fake((1 << 20) + 4), ok, ok, ok, ok, ok, null, ok, null, ok,
                                  ws, null) == -4


def test_varlen_allows_many_sequences(gdn):
    # packed sequences are bounded by their grids only: 4096 sequences x 32
    # value heads are accepted (the padded-batch entry point keeps B*H_v <= 65535)
    assert gdn.workspace_size_varlen(_shape(gdn, B=4096, T=40000)) > 0
    assert gdn.validate(_shape(gdn, B=4096, T=40000)) == -2
