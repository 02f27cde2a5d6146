"""gdn_chunk_fwd_noalloc (the forward whose workspace is the library's static
device scratch) against gdn_chunk_fwd on the same inputs, through the C ABI:
two calls in a row, the second on a smaller problem, each equal to the
allocating entry point's result bit for bit (the same kernels on the same
inputs) and within the bf16 bar of the fp64 oracle; problems too large for
the scratch array are refused before anything is launched."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import linear_attention_rnn_gdn_amd as g

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.lib()
    return g


def _cpu(x):
    return None if x is None else x.detach().cpu()


def _one(gdn, w, seed, ng):
    x = make_inputs(w, device="cuda", seed=seed)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    o = torch.full((w.B, w.T, w.Hv, w.dv), float("nan"), dtype=torch.float32, device="cuda")
    h = torch.full((w.B, w.Hv, w.dk, w.dv), float("nan"), dtype=torch.float32, device="cuda")
    gdn.chunk_fwd_noalloc(*args, out=o, final_state=h, chunk=w.chunk, n_groups=ng)
    torch.cuda.synchronize()
    o_ref, h_ref = gdn.chunk_fwd(*args, chunk=w.chunk, n_groups=ng)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(h, h_ref)
    oo, ho = oracle.fwd(**{kk: _cpu(vv) for kk, vv in x.items()})
    rms = float(np.sqrt(np.mean(oo ** 2)))
    tol = 2e-2 if w.dtype == "bf16" else 1e-4
    assert float(np.abs(o.cpu().numpy() - oo).max()) <= tol * rms
    assert float(np.abs(h.cpu().numpy() - ho).max()) <= tol * rms
    return o


def test_noalloc_equals_allocating_entry_point(gdn):
    # the 4096-token layer (the largest problem the scratch is sized for),
    # then a smaller, grouped problem reusing the same scratch
    w1 = WORKLOADS["qwen3next_8b_layer"]
    _one(gdn, w1, seed=61, ng=0)
    w2 = WORKLOADS["tiny"].replace(T=1000, Hqk=2, Hv=4, chunk=128, dtype="bf16", h0_std=0.05)
    _one(gdn, w2, seed=62, ng=4)


def test_noalloc_refuses_problems_beyond_the_scratch(gdn):
    w = WORKLOADS["qwen3next_8b_layer"].replace(T=65536)
    shape = gdn.make_shape(w.B, w.T, w.Hqk, w.Hv, 128, 128, 128, 0, torch.bfloat16, torch.float32)
    assert gdn.workspace_size(shape) > gdn.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(1 << 20)
    st = gdn.lib().gdn_chunk_fwd_noalloc(ctypes.byref(shape), fake, fake, fake, fake, fake, None, fake,
                                         None, None)
    assert st == -5
