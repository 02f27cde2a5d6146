"""MI355X-native Gated DeltaNet chunked forward.

A thin Python binding over ``libgdn.so`` (C ABI declared in include/gdn.h).
Every step of the computation runs in the library's HIP kernels; this module
only checks tensors, allocates outputs and workspace with torch and passes
device pointers plus torch's current HIP stream.  There is no fallback: if the
library is not built, every call raises.

Functions (same names as the C entry points, without the ``gdn_`` prefix):
  chunk_fwd(q, k, v, g, beta, h0=None, chunk=128, n_groups=0, ...) -> (o, h_T)
  chunk_fold(k, v, g, beta, n_groups, chunk=128)                 -> (A, Bm)
  compose_prefix(A, Bm, h_init=None, split_bf16=False)          -> (h_in, h_final)
  chunk_transform(k, v, g, beta, chunk=128, want_T=False)       -> (G, T, W, U)
  workspace_size(...), validate(...)
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

F32, BF16 = 0, 1
PREFIX_SPLIT_BF16, PREFIX_SEQUENTIAL, PREFIX_BLOCKED = 1, 2, 4
STATUS = {0: "ok", -1: "null pointer", -2: "unsupported or inconsistent sizes",
          -3: "unsupported dtype", -4: "misaligned pointer", -5: "workspace too small",
          -6: "kernel launch failed"}


class GdnShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "T", "H_qk", "H_v", "d_k", "d_v", "chunk", "n_groups", "dtype", "o_dtype")]


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {STATUS.get(status, status)} (status {status})")
        self.status = status


_lib = None

SYMBOLS = ("gdn_status_str", "gdn_validate", "gdn_workspace_size", "gdn_workspace_size_varlen",
           "gdn_chunk_fwd", "gdn_chunk_fwd_varlen",
           "gdn_chunk_fwd_stages", "gdn_chunk_fwd_timed", "gdn_chunk_fold", "gdn_compose_prefix",
           "gdn_chunk_transform", "gdn_chunk_fwd_noalloc", "gdn_chunk_fwd_affine",
           "gdn_workspace_size_bwd", "gdn_chunk_bwd_state", "gdn_workspace_size_bwd_grads", "gdn_chunk_bwd")
STAGE_PREP, STAGE_FOLD, STAGE_PREFIX, STAGE_WALK, STAGE_OUT, STAGE_ALL = 1, 2, 4, 8, 16, 31


def lib():
    """Load libgdn.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "(there is no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        P, I, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        SP = ctypes.POINTER(GdnShape)
        L.gdn_status_str.argtypes = [I]
        L.gdn_status_str.restype = ctypes.c_char_p
        L.gdn_validate.argtypes = [SP]
        L.gdn_validate.restype = I
        L.gdn_workspace_size.argtypes = [SP, ctypes.POINTER(SZ)]
        L.gdn_workspace_size.restype = I
        L.gdn_workspace_size_varlen.argtypes = [SP, ctypes.POINTER(SZ)]
        L.gdn_workspace_size_varlen.restype = I
        L.gdn_chunk_fwd_varlen.argtypes = [SP] + [P] * 10 + [SZ, P]
        L.gdn_chunk_fwd_varlen.restype = I
        L.gdn_chunk_fwd.argtypes = [SP] + [P] * 9 + [SZ, P]
        L.gdn_chunk_fwd.restype = I
        L.gdn_chunk_fwd_stages.argtypes = [SP, I] + [P] * 9 + [SZ, P]
        L.gdn_chunk_fwd_stages.restype = I
        L.gdn_chunk_fwd_timed.argtypes = [SP, I] + [P] * 9 + [SZ, P, P, P]
        L.gdn_chunk_fwd_timed.restype = I
        L.gdn_chunk_fold.argtypes = [SP] + [P] * 7 + [SZ, P]
        L.gdn_chunk_fold.restype = I
        L.gdn_compose_prefix.argtypes = [I, I, I, I] + [P] * 5 + [I, P]
        L.gdn_compose_prefix.restype = I
        L.gdn_chunk_transform.argtypes = [SP] + [P] * 8 + [P]
        L.gdn_chunk_transform.restype = I
        L.gdn_chunk_fwd_noalloc.argtypes = [SP] + [P] * 9
        L.gdn_chunk_fwd_noalloc.restype = I
        L.gdn_chunk_fwd_affine.argtypes = [SP] + [P] * 10 + [SZ, P]
        L.gdn_chunk_fwd_affine.restype = I
        L.gdn_workspace_size_bwd.argtypes = [SP, ctypes.POINTER(SZ)]
        L.gdn_workspace_size_bwd.restype = I
        L.gdn_chunk_bwd_state.argtypes = [SP] + [P] * 9 + [SZ, P]
        L.gdn_chunk_bwd_state.restype = I
        L.gdn_workspace_size_bwd_grads.argtypes = [SP, ctypes.POINTER(SZ)]
        L.gdn_workspace_size_bwd_grads.restype = I
        L.gdn_chunk_bwd.argtypes = [SP] + [P] * 15 + [SZ, P]
        L.gdn_chunk_bwd.restype = I
        _lib = L
    return _lib


def _check(st: int, where: str):
    if st != 0:
        raise GdnError(st, where)


def _dt(t: torch.dtype) -> int:
    if t == torch.float32:
        return F32
    if t == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t}")


def make_shape(B, T, H_qk, H_v, d_k=128, d_v=128, chunk=128, n_groups=0,
               dtype=torch.bfloat16, o_dtype=torch.float32) -> GdnShape:
    return GdnShape(B, T, H_qk, H_v, d_k, d_v, chunk, n_groups, _dt(dtype), _dt(o_dtype))


def validate(shape: GdnShape) -> int:
    """Host-only check; returns the status code (0 = supported)."""
    return int(lib().gdn_validate(ctypes.byref(shape)))


def workspace_size(shape: GdnShape) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().gdn_workspace_size(ctypes.byref(shape), ctypes.byref(n)), "gdn_workspace_size")
    return int(n.value)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _inputs(q, k, v, g, beta):
    B, T, Hqk, dk = k.shape
    Hv, dv = v.shape[2], v.shape[3]
    dev = k.device
    if q is not None:
        _need(q, "q", k.dtype, (B, T, Hqk, dk), dev)
    _need(k, "k", None, None, dev)
    _need(v, "v", k.dtype, (B, T, Hv, dv), dev)
    _need(g, "g", torch.float32, (B, T, Hv), dev)
    _need(beta, "beta", torch.float32, (B, T, Hv), dev)
    return B, T, Hqk, Hv, dk, dv, dev


def chunk_fwd(q, k, v, g, beta, h0=None, chunk=128, n_groups=0, o_dtype=torch.float32,
              output_final_state=True, workspace=None, out=None, final_state=None, stream=None,
              stages=None, events=None):
    """Gated DeltaNet chunked forward (gdn_chunk_fwd; gdn_chunk_fwd_stages when
    ``stages`` is a mask of STAGE_* bits; gdn_chunk_fwd_timed when ``events`` =
    (starts, stops) gives, per stage bit b = 0..4, timing torch.cuda.Event
    objects (already recorded once, so that they exist) or None).

    q, k [B,T,H_qk,d_k]; v [B,T,H_v,d_v] (bf16 or fp32); g, beta [B,T,H_v] fp32;
    h0 [B,H_v,d_k,d_v] fp32 or None.  Returns (o [B,T,H_v,d_v] o_dtype, h_T or None)."""
    B, T, Hqk, Hv, dk, dv, dev = _inputs(q, k, v, g, beta)
    shape = make_shape(B, T, Hqk, Hv, dk, dv, chunk, n_groups, k.dtype, o_dtype)
    if h0 is not None:
        _need(h0, "h0", torch.float32, (B, Hv, dk, dv), dev)
    need = workspace_size(shape)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    o = out if out is not None else torch.empty((B, T, Hv, dv), dtype=o_dtype, device=dev)
    _need(o, "o", o_dtype, (B, T, Hv, dv), dev)
    hT = None
    if output_final_state:
        hT = final_state if final_state is not None else torch.empty((B, Hv, dk, dv),
                                                                    dtype=torch.float32, device=dev)
        _need(hT, "h_T", torch.float32, (B, Hv, dk, dv), dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT),
            _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(stream))
    if events is not None:
        arr = [(ctypes.c_void_p * 5)(*[e.cuda_event if e is not None else None for e in evs])
               for evs in events]
        _check(lib().gdn_chunk_fwd_timed(ctypes.byref(shape), int(STAGE_ALL if stages is None else stages),
                                         *args, arr[0], arr[1]), "gdn_chunk_fwd_timed")
    elif stages is None:
        _check(lib().gdn_chunk_fwd(ctypes.byref(shape), *args), "gdn_chunk_fwd")
    else:
        _check(lib().gdn_chunk_fwd_stages(ctypes.byref(shape), int(stages), *args),
               "gdn_chunk_fwd_stages")
    return o, hT


NOALLOC_SCRATCH_BYTES = 256 << 20


def chunk_fwd_noalloc(q, k, v, g, beta, h0, out, final_state=None, chunk=128, n_groups=0,
                      stream=None):
    """gdn_chunk_fwd_noalloc: the forward with the library's static device
    scratch as its workspace (nothing is allocated by the library; the caller
    passes the outputs).  out [B,T,H_v,d_v] (fp32 or bf16: the output dtype),
    final_state [B,H_v,d_k,d_v] fp32 or None.  Returns (out, final_state)."""
    B, T, Hqk, Hv, dk, dv, dev = _inputs(q, k, v, g, beta)
    _need(out, "o", None, (B, T, Hv, dv), dev)
    shape = make_shape(B, T, Hqk, Hv, dk, dv, chunk, n_groups, k.dtype, out.dtype)
    if h0 is not None:
        _need(h0, "h0", torch.float32, (B, Hv, dk, dv), dev)
    if final_state is not None:
        _need(final_state, "h_T", torch.float32, (B, Hv, dk, dv), dev)
    _check(lib().gdn_chunk_fwd_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                       _ptr(h0), _ptr(out), _ptr(final_state), _stream(stream)),
           "gdn_chunk_fwd_noalloc")
    return out, final_state


def chunk_fwd_affine(q, k, v, g, beta, h0=None, chunk=128, o_dtype=torch.float32, workspace=None,
                     out=None, final_state=None, affine=None, stream=None):
    """The forward that also returns the affine map of the whole sequence
    (gdn_chunk_fwd_affine): (o, h_T, A) with A [B,H_v,d_k,d_k] fp32 and
    h_T = A h0 + B (B = h_T when h0 is None)."""
    B, T, Hqk, Hv, dk, dv, dev = _inputs(q, k, v, g, beta)
    shape = make_shape(B, T, Hqk, Hv, dk, dv, chunk, 0, k.dtype, o_dtype)
    if h0 is not None:
        _need(h0, "h0", torch.float32, (B, Hv, dk, dv), dev)
    need = workspace_size(shape)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    o = out if out is not None else torch.empty((B, T, Hv, dv), dtype=o_dtype, device=dev)
    _need(o, "o", o_dtype, (B, T, Hv, dv), dev)
    hT = final_state if final_state is not None else torch.empty((B, Hv, dk, dv), dtype=torch.float32, device=dev)
    _need(hT, "h_T", torch.float32, (B, Hv, dk, dv), dev)
    A = affine if affine is not None else torch.empty((B, Hv, dk, dk), dtype=torch.float32, device=dev)
    _need(A, "A", torch.float32, (B, Hv, dk, dk), dev)
    _check(lib().gdn_chunk_fwd_affine(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                      _ptr(h0), _ptr(o), _ptr(hT), _ptr(A), _ptr(workspace),
                                      ctypes.c_size_t(workspace.numel()), _stream(stream)),
           "gdn_chunk_fwd_affine")
    return o, hT, A


def chunk_bwd_state(q, k, g, beta, dO, dh_T=None, chunk=128, want_chunks=True, workspace=None, stream=None):
    """The chunked backward's state cotangents (gdn_chunk_bwd_state): the
    reverse chunk walk dh_n = e^{G_last} dh_{n+1} - W^T (K_g dh_{n+1}) + ddh_n
    from dh_T.  q, k [B,T,H_qk,d_k]; g, beta [B,T,H_v] fp32; dO [B,T,H_v,d_v]
    fp32; dh_T [B,H_v,d_k,d_v] fp32 or None.  Returns (dh_chunks
    [B,H_v,N,d_k,d_v] or None, dh0 [B,H_v,d_k,d_v])."""
    B, T, Hqk, dk = k.shape
    Hv, dv = dO.shape[2], dO.shape[3]
    dev = k.device
    _need(q, "q", k.dtype, (B, T, Hqk, dk), dev)
    _need(k, "k", None, None, dev)
    _need(g, "g", torch.float32, (B, T, Hv), dev)
    _need(beta, "beta", torch.float32, (B, T, Hv), dev)
    _need(dO, "dO", torch.float32, (B, T, Hv, dv), dev)
    if dh_T is not None:
        _need(dh_T, "dh_T", torch.float32, (B, Hv, dk, dv), dev)
    shape = make_shape(B, T, Hqk, Hv, dk, dv, chunk, 0, k.dtype, torch.float32)
    n = ctypes.c_size_t(0)
    _check(lib().gdn_workspace_size_bwd(ctypes.byref(shape), ctypes.byref(n)), "gdn_workspace_size_bwd")
    if workspace is None:
        workspace = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=dev)
    N = -(-T // chunk)
    dhc = torch.empty((B, Hv, N, dk, dv), dtype=torch.float32, device=dev) if want_chunks else None
    dh0 = torch.empty((B, Hv, dk, dv), dtype=torch.float32, device=dev)
    _check(lib().gdn_chunk_bwd_state(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(g), _ptr(beta), _ptr(dO),
                                     _ptr(dh_T), _ptr(dhc), _ptr(dh0), _ptr(workspace),
                                     ctypes.c_size_t(workspace.numel()), _stream(stream)),
           "gdn_chunk_bwd_state")
    return dhc, dh0


def workspace_size_bwd_grads(shape: GdnShape) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().gdn_workspace_size_bwd_grads(ctypes.byref(shape), ctypes.byref(n)), "gdn_workspace_size_bwd_grads")
    return int(n.value)


def chunk_bwd(q, k, v, g, beta, dO, h0=None, dh_T=None, chunk=128, workspace=None, out=None, stream=None):
    """Gradients of sum_t <o_t, dO_t> + <h_T, dh_T> through the chunked
    forward (gdn_chunk_bwd).  q, k [B,T,H_qk,d_k]; v [B,T,H_v,d_v]; g, beta
    [B,T,H_v] fp32; dO [B,T,H_v,d_v] fp32; h0, dh_T [B,H_v,d_k,d_v] fp32 or
    None.  Returns a dict of fp32 tensors dq, dk [B,T,H_qk,d_k], dv
    [B,T,H_v,d_v], dg, dbeta [B,T,H_v], dh0 [B,H_v,d_k,d_v] (``out``: such a
    dict to write into)."""
    B, T, Hqk, Hv, dk, dv, dev = _inputs(q, k, v, g, beta)
    _need(dO, "dO", torch.float32, (B, T, Hv, dv), dev)
    for name, x in (("h0", h0), ("dh_T", dh_T)):
        if x is not None:
            _need(x, name, torch.float32, (B, Hv, dk, dv), dev)
    shape = make_shape(B, T, Hqk, Hv, dk, dv, chunk, 0, q.dtype, torch.float32)
    if workspace is None:
        workspace = torch.empty(max(workspace_size_bwd_grads(shape), 1), dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    want = dict(dq=(B, T, Hqk, dk), dk=(B, T, Hqk, dk), dv=(B, T, Hv, dv), dg=(B, T, Hv), dbeta=(B, T, Hv),
                dh0=(B, Hv, dk, dv))
    if out is None:
        out = {kk: torch.empty(sh, **f32) for kk, sh in want.items()}
    for kk, sh in want.items():
        _need(out[kk], kk, torch.float32, sh, dev)
    _check(lib().gdn_chunk_bwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                               _ptr(dO), _ptr(dh_T), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                               _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["dh0"]), _ptr(workspace),
                               ctypes.c_size_t(workspace.numel()), _stream(stream)), "gdn_chunk_bwd")
    return out


def workspace_size_varlen(shape: GdnShape) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().gdn_workspace_size_varlen(ctypes.byref(shape), ctypes.byref(n)), "gdn_workspace_size_varlen")
    return int(n.value)


def chunk_fwd_varlen(q, k, v, g, beta, cu_seqlens, h0=None, chunk=128, o_dtype=torch.float32,
                     output_final_state=True, workspace=None, out=None, final_state=None, stream=None):
    """Chunked forward over packed variable-length sequences
    (gdn_chunk_fwd_varlen).  q, k [1,T,H_qk,d_k]; v [1,T,H_v,d_v]; g, beta
    [1,T,H_v]; cu_seqlens int32 [n+1] on the device, or a Python sequence of
    the n+1 offsets (sequence s = tokens cu[s]..cu[s+1]); h0 [n,H_v,d_k,d_v]
    or None.  Returns (o, h_T [n,...] or None)."""
    B, T, Hqk, Hv, dk, dv, dev = _inputs(q, k, v, g, beta)
    if B != 1:
        raise ValueError("packed sequences: the batch dimension of q, k, v, g, beta must be 1")
    if not isinstance(cu_seqlens, torch.Tensor):   # a sequence of offsets
        cu_seqlens = torch.tensor(list(cu_seqlens), dtype=torch.int32, device=dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, None, dev)
    nseq = cu_seqlens.numel() - 1
    if nseq < 1:
        raise ValueError("cu_seqlens must hold at least two offsets")
    shape = make_shape(nseq, T, Hqk, Hv, dk, dv, chunk, 0, k.dtype, o_dtype)
    if h0 is not None:
        _need(h0, "h0", torch.float32, (nseq, Hv, dk, dv), dev)
    need = workspace_size_varlen(shape)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    o = out if out is not None else torch.empty((1, T, Hv, dv), dtype=o_dtype, device=dev)
    _need(o, "o", o_dtype, (1, T, Hv, dv), dev)
    hT = None
    if output_final_state:
        hT = final_state if final_state is not None else torch.empty((nseq, Hv, dk, dv),
                                                                    dtype=torch.float32, device=dev)
        _need(hT, "h_T", torch.float32, (nseq, Hv, dk, dv), dev)
    _check(lib().gdn_chunk_fwd_varlen(ctypes.byref(shape), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT), _ptr(workspace),
                                      ctypes.c_size_t(workspace.numel()), _stream(stream)),
           "gdn_chunk_fwd_varlen")
    return o, hT


def chunk_fold(k, v, g, beta, n_groups, chunk=128, workspace=None, stream=None):
    """Per-group affine pairs (gdn_chunk_fold): A [B,H_v,G,d_k,d_k], Bm [B,H_v,G,d_k,d_v]."""
    B, T, Hqk, Hv, dk, dv, dev = _inputs(None, k, v, g, beta)
    shape = make_shape(B, T, Hqk, Hv, dk, dv, chunk, n_groups, k.dtype, torch.float32)
    Gn = max(int(n_groups), 1)
    need = workspace_size(shape)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    A = torch.empty((B, Hv, Gn, dk, dk), dtype=torch.float32, device=dev)
    Bm = torch.empty((B, Hv, Gn, dk, dv), dtype=torch.float32, device=dev)
    st = lib().gdn_chunk_fold(ctypes.byref(shape), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A),
                              _ptr(Bm), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
                              _stream(stream))
    _check(st, "gdn_chunk_fold")
    return A, Bm


def compose_prefix(A, Bm, h_init=None, split_bf16=False, want_h_in=True, stream=None, form=None):
    """Exclusive prefix of affine pairs (gdn_compose_prefix).  ``form``: None
    lets the library choose, "sequential" or "blocked" force one.
    A [BH,n,d_k,d_k], Bm [BH,n,d_k,d_v] fp32; h_init [BH,d_k,d_v] or None.
    Returns (h_in [BH,n,d_k,d_v] or None, h_final [BH,d_k,d_v])."""
    BH, n, dk, _ = A.shape
    dv = Bm.shape[3]
    dev = A.device
    _need(A, "A", torch.float32, None, dev)
    _need(Bm, "Bm", torch.float32, (BH, n, dk, dv), dev)
    if h_init is not None:
        _need(h_init, "h_init", torch.float32, (BH, dk, dv), dev)
    h_in = torch.empty((BH, n, dk, dv), dtype=torch.float32, device=dev) if want_h_in else None
    h_fin = torch.empty((BH, dk, dv), dtype=torch.float32, device=dev)
    st = lib().gdn_compose_prefix(BH, n, dk, dv, _ptr(A), _ptr(Bm), _ptr(h_init), _ptr(h_in),
                                  _ptr(h_fin), (PREFIX_SPLIT_BF16 if split_bf16 else 0) |
                                  {None: 0, "sequential": PREFIX_SEQUENTIAL,
                                   "blocked": PREFIX_BLOCKED}[form],
                                  _stream(stream))
    _check(st, "gdn_compose_prefix")
    return h_in, h_fin


def chunk_transform(k, v, g, beta, chunk=128, want_T=False, stream=None):
    """Intra-chunk transform (gdn_chunk_transform): G [B,H_v,N,C], T [B,H_v,N,C,C] or None,
    W [B,H_v,N,C,d_k], U [B,H_v,N,C,d_v], all fp32."""
    B, T, Hqk, Hv, dk, dv, dev = _inputs(None, k, v, g, beta)
    shape = make_shape(B, T, Hqk, Hv, dk, dv, chunk, 0, k.dtype, torch.float32)
    _check(validate(shape), "gdn_chunk_transform")
    N = -(-T // chunk)   # a partial last chunk is padded with identity steps
    f = dict(dtype=torch.float32, device=dev)
    G = torch.empty((B, Hv, N, chunk), **f)
    Tm = torch.empty((B, Hv, N, chunk, chunk), **f) if want_T else None
    W = torch.empty((B, Hv, N, chunk, dk), **f)
    U = torch.empty((B, Hv, N, chunk, dv), **f)
    st = lib().gdn_chunk_transform(ctypes.byref(shape), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                   _ptr(G), _ptr(Tm), _ptr(W), _ptr(U), _stream(stream))
    _check(st, "gdn_chunk_transform")
    return G, Tm, W, U
