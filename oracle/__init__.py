"""fp64 CPU oracle for the Gated DeltaNet chunked forward.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the product package
``linear_attention_rnn_gdn_amd`` never does, and the two share no code.

Two halves:

* ``gdn_oracle.c`` (loaded here through ctypes): the per-token rule, the
  per-group affine fold and the exclusive prefix, all in fp64, written from
  their plain definitions (see that file's header).
* ``chunked.py``: the chunk-level quantities of the method in numpy fp64 --
  decay cumsum, the gated strict-lower beta*K*K^T matrix, its unit-triangular
  inverse by forward substitution, the WY pair (W, U), the per-chunk affine
  pair (A, B) and the chunk output.  These give the values each hot-path step
  must reproduce and, run end to end, an independent evaluation of the rule
  used to pin the per-token oracle.
* ``backward.py``: the gradient of the per-token rule with respect to q, k,
  v, g, beta and h0 (reverse-mode differentiation written out token by
  token, numpy fp64), the reference for a backward pass.

Parity status: every function here is pinned by a CPU test against closed
forms, invariants, finite differences or an independent algorithm
(tests/test_oracle_*.py); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import chunked  # noqa: F401  (re-exported)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")
SRC_PATH = os.path.join(_HERE, "gdn_oracle.c")

F32, BF16 = 0, 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into oracle/libgdn_oracle.so."""
    import subprocess

    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", SRC_PATH, "-o", tmp, "-lm"]
        )
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.gdn_oracle_fwd.argtypes = [I] * 7 + [P] * 6 + [I] * 4 + [P, P, I]
        lib.gdn_oracle_fwd.restype = I
        lib.gdn_oracle_fold.argtypes = [I] * 8 + [P] * 6 + [I]
        lib.gdn_oracle_fold.restype = I
        lib.gdn_oracle_prefix.argtypes = [I] * 4 + [P] * 5
        lib.gdn_oracle_prefix.restype = I
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _raw(x):
    """Return (contiguous numpy array of the stored bits, dtype code).

    Accepts numpy float32 arrays, or torch CPU tensors of dtype float32 /
    bfloat16 (bf16 is passed as its raw 16-bit words so the C side widens the
    exact rounded values)."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy(), BF16
            if x.dtype == torch.float32:
                return x.numpy(), F32
            raise TypeError(f"oracle: unsupported tensor dtype {x.dtype}")
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    raise TypeError(f"oracle: unsupported array dtype {x.dtype}")


def _f32(x):
    if x is None:
        return None
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().cpu().float().numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def fwd(q, k, v, g, beta, h0=None, heads=None, cols=None, want_o=True, nthreads=None):
    """Per-token rule in fp64 (gdn_oracle.c: gdn_oracle_fwd).

    q, k [B,T,Hqk,dk]; v [B,T,Hv,dv] (fp32 or bf16); g, beta [B,T,Hv] fp32;
    h0 [B,Hv,dk,dv] fp32 or None.  ``heads``=(lo,hi) and ``cols``=(lo,hi)
    restrict the value heads and state columns computed.
    Returns (o [B,T,nh,nc] fp64 or None, hT [B,nh,dk,nc] fp64)."""
    qr, dt = _raw(q)
    kr, dt2 = _raw(k)
    vr, dt3 = _raw(v)
    if not (dt == dt2 == dt3):
        raise TypeError("oracle: q, k, v must share a dtype")
    B, T, Hqk, dk = qr.shape
    Hv, dv = vr.shape[2], vr.shape[3]
    gr, br, hr = _f32(g), _f32(beta), _f32(h0)
    hlo, hhi = heads if heads is not None else (0, Hv)
    clo, chi = cols if cols is not None else (0, dv)
    nh, nc = hhi - hlo, chi - clo
    o = np.empty((B, T, nh, nc), np.float64) if want_o else None
    hT = np.empty((B, nh, dk, nc), np.float64)
    rc = _load().gdn_oracle_fwd(
        B, T, Hqk, Hv, dk, dv, dt, _ptr(qr), _ptr(kr), _ptr(vr), _ptr(gr), _ptr(br), _ptr(hr),
        hlo, hhi, clo, chi, _ptr(o), _ptr(hT), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("gdn_oracle_fwd: bad arguments")
    return o, hT


def fold(k, v, g, beta, n_groups, nthreads=None):
    """Per-group affine pairs in fp64 (gdn_oracle.c: gdn_oracle_fold).
    Returns A [B,Hv,G,dk,dk], Bm [B,Hv,G,dk,dv]."""
    kr, dt = _raw(k)
    vr, dt2 = _raw(v)
    if dt != dt2:
        raise TypeError("oracle: k, v must share a dtype")
    B, T, Hqk, dk = kr.shape
    Hv, dv = vr.shape[2], vr.shape[3]
    gr, br = _f32(g), _f32(beta)
    A = np.empty((B, Hv, n_groups, dk, dk), np.float64)
    Bm = np.empty((B, Hv, n_groups, dk, dv), np.float64)
    rc = _load().gdn_oracle_fold(
        B, T, Hqk, Hv, dk, dv, dt, int(n_groups), _ptr(kr), _ptr(vr), _ptr(gr), _ptr(br),
        _ptr(A), _ptr(Bm), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("gdn_oracle_fold: bad arguments")
    return A, Bm


def prefix(A, Bm, h_init=None):
    """Exclusive prefix of affine pairs in fp64 (gdn_oracle.c: gdn_oracle_prefix).
    A [BH,n,dk,dk], Bm [BH,n,dk,dv] (taken as fp32, as the GPU receives them),
    h_init [BH,dk,dv] or None.  Returns (h_in [BH,n,dk,dv], h_final [BH,dk,dv])."""
    Ar, Br, hr = _f32(A), _f32(Bm), _f32(h_init)
    BH, n, dk, _ = Ar.shape
    dv = Br.shape[3]
    h_in = np.empty((BH, n, dk, dv), np.float64)
    h_fin = np.empty((BH, dk, dv), np.float64)
    rc = _load().gdn_oracle_prefix(BH, n, dk, dv, _ptr(Ar), _ptr(Br), _ptr(hr), _ptr(h_in),
                                   _ptr(h_fin))
    if rc != 0:
        raise ValueError("gdn_oracle_prefix: bad arguments")
    return h_in, h_fin
