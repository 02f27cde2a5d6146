"""Seeded synthetic workloads for the Gated DeltaNet chunked forward.

This module holds the workload shapes and the seeded input draws only; it
contains none of the method's arithmetic and is shared by the tests, the
benchmark and the smoke check (both the HIP path and the oracle read the
same tensors).

Draws (fixed order q, k, v, beta, g, h0, one seeded torch generator):
  q, k  ~ N(0, 1), then divided by their L2 norm over d_k (no epsilon),
        then cast to the workload dtype;
  v     ~ N(0, 1), cast to the workload dtype;
  beta  = sigmoid(N(0, 1))                     fp32
  g     = log(sigmoid(N(3, 1)))                fp32 (per-token log decay, <= 0)
  h0    ~ N(0, 0.02^2) i.i.d. or zero          fp32
Layouts: q, k [B,T,Hqk,dk]; v [B,T,Hv,dv]; g, beta [B,T,Hv]; h0 [B,Hv,dk,dv].

The pages measure whole-model training on TPUs with synthetic data and name no
public dataset; these draws stand in for the activations of a GDN layer at the
shapes those runs use (Qwen3-Next dense-8B-shaped: 16 query/key heads, 32
value heads, head dim 128, sequence 4096; dense GDN model at d_model 4096:
32 heads, sequence 8192; context-parallel runs at 262,144 and 1,048,576
tokens; chunk 128).
"""
from __future__ import annotations

import dataclasses

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    Hqk: int
    Hv: int
    dk: int
    dv: int
    chunk: int
    n_groups: int          # 0/1 = one sequential walk; >1 = fold / prefix / replay
    dtype: str             # "f32" or "bf16": dtype of q, k, v (and o)
    h0_std: float          # 0 = zero initial state
    desc: str

    @property
    def tokens(self) -> int:
        return self.B * self.T

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 512, 2, 2, 128, 128, 64, 1, "f32", 0.0,
                     "tiny GDN forward, B=1 H=2 T=512, chunk 64, fp32"),
    "qwen3next_8b_layer": Workload("qwen3next_8b_layer", 1, 4096, 16, 32, 128, 128, 128, 1,
                                   "bf16", 0.02,
                                   "Qwen3-Next-8B-shaped GDN layer, B=1 T=4096, 16 qk / 32 v "
                                   "heads, chunk 128, bf16, h0~N(0,0.02)"),
    "dense_d4096_layer": Workload("dense_d4096_layer", 2, 8192, 32, 32, 128, 128, 128, 1,
                                  "bf16", 0.0,
                                  "dense GDN layer at d_model 4096, B=2 T=8192, 32 heads, "
                                  "chunk 128, bf16"),
    "long_256k": Workload("long_256k", 1, 262144, 32, 32, 128, 128, 128, 256, "bf16", 0.0,
                          "long sequence T=262144, 32 heads, chunk 128, 256 chunk-groups, bf16"),
    "million_1m": Workload("million_1m", 1, 1048576, 16, 32, 128, 128, 128, 256, "bf16", 0.02,
                           "million-token sequence T=1048576, 16 qk / 32 v heads, chunk 128, "
                           "256 chunk-groups, bf16, h0~N(0,0.02)"),
}

ORDER = ["tiny", "qwen3next_8b_layer", "dense_d4096_layer", "long_256k", "million_1m"]


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def default_seed(w: Workload) -> int:
    return 1000 + ORDER.index(w.name) if w.name in ORDER else 1000


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


@torch.no_grad()
def make_inputs(w: Workload, device="cpu", seed=None, t_block: int = 65536,
                g_const=None, beta_scale=None):
    """Draw the workload's inputs on ``device`` (seeded, deterministic per device).

    Large T is drawn in blocks of ``t_block`` tokens to bound temporaries.
    ``g_const`` (e.g. 0.0) replaces the decay draw by a constant and
    ``beta_scale`` multiplies beta: weak-decay variants in which a group's
    affine map stays far from zero, used by the composition tests."""
    seed = default_seed(w) if seed is None else int(seed)
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    dt = torch_dtype(w.dtype)
    B, T, Hqk, Hv, dk, dv = w.B, w.T, w.Hqk, w.Hv, w.dk, w.dv
    q = torch.empty((B, T, Hqk, dk), dtype=dt, device=dev)
    k = torch.empty((B, T, Hqk, dk), dtype=dt, device=dev)
    v = torch.empty((B, T, Hv, dv), dtype=dt, device=dev)
    beta = torch.empty((B, T, Hv), dtype=torch.float32, device=dev)
    g = torch.empty((B, T, Hv), dtype=torch.float32, device=dev)
    for name, dst, width, unit in (("q", q, (Hqk, dk), True), ("k", k, (Hqk, dk), True),
                                   ("v", v, (Hv, dv), False)):
        for b in range(B):
            for s in range(0, T, t_block):
                e = min(T, s + t_block)
                x = torch.randn((e - s,) + width, generator=gen, device=dev, dtype=torch.float32)
                if unit:
                    x = _unit_rows(x)
                dst[b, s:e] = x.to(dt)
    for b in range(B):
        for s in range(0, T, t_block):
            e = min(T, s + t_block)
            beta[b, s:e] = torch.sigmoid(
                torch.randn((e - s, Hv), generator=gen, device=dev, dtype=torch.float32))
    for b in range(B):
        for s in range(0, T, t_block):
            e = min(T, s + t_block)
            x = torch.randn((e - s, Hv), generator=gen, device=dev, dtype=torch.float32) + 3.0
            g[b, s:e] = torch.nn.functional.logsigmoid(x)
    if w.h0_std > 0:
        h0 = torch.randn((B, Hv, dk, dv), generator=gen, device=dev,
                         dtype=torch.float32) * w.h0_std
    else:
        h0 = None
    if g_const is not None:
        g.fill_(float(g_const))
    if beta_scale is not None:
        beta.mul_(float(beta_scale))
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0)


# Packed variable-length sequences: n_seq sequences, lengths drawn uniformly
# from [1, max_len] with their own seeded generator, concatenated along one
# row (B = 1) and drawn as one workload of their total length; one h0 per
# sequence, N(0, h0_std^2).
PACKED = {
    "packed_8b_mix": dict(n_seq=16, max_len=8192, Hqk=16, Hv=32, chunk=128, dtype="bf16",
                          h0_std=0.02, seed=2000,
                          desc="16 packed sequences of 1..8192 tokens, Qwen3-Next-8B-shaped "
                               "heads (16 qk / 32 v), chunk 128, bf16, h0~N(0,0.02) each"),
}


@torch.no_grad()
def make_packed_inputs(name: str, device="cpu"):
    """Inputs of a packed workload: the tensors of make_inputs over the total
    length (B = 1), cu_seqlens (int32) and per-sequence h0."""
    p = PACKED[name]
    gen = torch.Generator().manual_seed(p["seed"])
    lens = torch.randint(1, p["max_len"] + 1, (p["n_seq"],), generator=gen)
    cu = torch.zeros(p["n_seq"] + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(lens, 0).to(torch.int32)
    T = int(cu[-1])
    w = Workload(name, 1, T, p["Hqk"], p["Hv"], 128, 128, p["chunk"], 1, p["dtype"], 0.0, p["desc"])
    x = make_inputs(w, device=device, seed=p["seed"] + 1)
    h0 = torch.randn((p["n_seq"], p["Hv"], 128, 128), generator=gen) * p["h0_std"]
    x["h0"] = h0.to(device)
    return w, x, cu.to(device)

