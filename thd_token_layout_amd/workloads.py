"""Seeded synthetic workloads for the THD token-layout and gradient-return path.

This module only draws inputs: document lengths (hence cu_seqlens), shapes and
random tensor values.  It contains none of the layout or reduction arithmetic,
so the library tests and the CPU oracle can both be fed from it.

Shapes follow the pages' workloads: the gradient-return shape is the one of the
four-GB200 Megatron CP=4 run described in "Add stream-ordered CP gradient
return primitive" (section "Validation": S=262144, 20 heads, head dimension
128); the partition workloads use packed documents of mixed length as in
"[PyTorch] Add experimental packed-contiguous THD all-gather CP" (section
"Why": uneven packed documents).  No dataset is used: synthetic values stand in
for the training data of that run.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

DCS = "dual_chunk_swap"
PC = "packed_contiguous"


@dataclass(frozen=True)
class Workload:
    name: str
    policy: str            # ownership policy of the token layout
    cp_size: int           # W
    total_tokens: int      # T (or S)
    heads: int             # H
    head_dim: int          # D
    dtype: str             # "f32" or "bf16": element type of the inputs
    out_dtype: str         # element type of gradient-return outputs
    doc_lengths: str       # "fixed", "loguniform_x8", "uniform_1_4096", "single"
    value_dist: str        # "uniform_pm1" or "normal"
    value_std: float
    seed: int
    n_tensors: int         # Q,K,V -> 3; dK,dV -> 2
    kind: str              # "layout", "grad_return", "fused", "sweep"
    fixed_lengths: tuple = field(default=())
    description: str = ""

    @property
    def row_elems(self) -> int:
        return self.heads * self.head_dim


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_w2", DCS, 2, 48, 2, 8, "f32", "f32", "fixed", "uniform_pm1", 1.0, 1, 2,
                 "layout", fixed_lengths=(8, 16, 24),
                 description="W=2, documents {8,16,24}, [48,2,8] fp32 U[-1,1); partition, "
                             "gather and a 2-writer dK/dV gradient return"),
        Workload("dcs_t32k_w4", DCS, 4, 32768, 8, 128, "bf16", "bf16", "loguniform_x8", "normal",
                 1.0, 2, 3, "layout",
                 description="DualChunkSwap W=4, T=32768, log-uniform lengths in [256,8192] "
                             "rounded to multiples of 8, Q,K,V [T,8,128] bf16 N(0,1)"),
        Workload("pc_t64k_w4", PC, 4, 65536, 8, 128, "bf16", "bf16", "uniform_1_4096", "normal",
                 1.0, 3, 3, "layout",
                 description="packed-contiguous W=4, T=65536, lengths U{1..4096}, "
                             "Q,K,V [T,8,128] bf16 N(0,1)"),
        Workload("grad_s256k_w4", DCS, 4, 262144, 20, 128, "f32", "f32", "single", "normal",
                 1e-3, 4, 2, "grad_return",
                 description="owner gradient return W=4, S=262144, 4 writers x {dK,dV} "
                             "[S,20,128] fp32 N(0,1e-3), one document (two-chunk layout)"),
        Workload("fused_s128k_w8", DCS, 8, 131072, 32, 128, "bf16", "bf16", "single", "normal",
                 1e-3, 5, 2, "fused",
                 description="fused scatter+sum W=8, S=131072, 8 writers x {dK,dV} "
                             "[S,32,128] bf16 N(0,1e-3), fp32 accumulation, bf16 output"),
        Workload("sweep_w8", DCS, 8, 0, 1, 1, "f32", "f32", "single", "normal", 1.0, 6, 1, "sweep",
                 description="W=8 fp32 slot buffers of 1 KiB .. 16 MiB summed into one"),
        Workload("dcs_s256k_w4", DCS, 4, 262144, 20, 128, "bf16", "bf16", "loguniform_x8",
                 "normal", 1.0, 7, 3, "layout",
                 description="DualChunkSwap W=4 at S=262144, lengths as dcs_t32k_w4, "
                             "Q,K,V [S,20,128] bf16 N(0,1)"),
        Workload("pc_s256k_w4", PC, 4, 262144, 20, 128, "bf16", "bf16", "uniform_1_4096",
                 "normal", 1.0, 8, 3, "layout",
                 description="packed-contiguous W=4 at S=262144, lengths as pc_t64k_w4, "
                             "Q,K,V [S,20,128] bf16 N(0,1)"),
        Workload("dcs1_s256k_w4", DCS, 4, 262144, 20, 128, "bf16", "bf16", "single", "normal",
                 1.0, 9, 3, "layout",
                 description="DualChunkSwap W=4, one document [0,262144], Q,K,V [S,20,128] bf16"),
    ]
}

SWEEP_BYTES = [1024 << k for k in range(15)]  # 1 KiB .. 16 MiB


def doc_lengths(kind: str, total_tokens: int, seed: int, fixed=()) -> List[int]:
    """Draw document lengths summing to total_tokens (last one truncated)."""
    if kind == "fixed":
        assert sum(fixed) == total_tokens
        return list(fixed)
    if kind == "single":
        return [total_tokens]
    rng = np.random.default_rng(seed)
    lengths: List[int] = []
    used = 0
    while used < total_tokens:
        if kind == "loguniform_x8":
            u = rng.uniform(np.log(256.0), np.log(8192.0))
            length = 8 * int(np.floor(np.exp(u) / 8.0 + 0.5))
            length = min(max(length, 256), 8192)
        elif kind == "uniform_1_4096":
            length = int(rng.integers(1, 4097))
        else:
            raise ValueError(kind)
        length = min(length, total_tokens - used)
        lengths.append(length)
        used += length
    return lengths


def cu_from_lengths(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def cu_seqlens(w: Workload) -> np.ndarray:
    return cu_from_lengths(doc_lengths(w.doc_lengths, w.total_tokens, w.seed, w.fixed_lengths))


def random_tensors(w: Workload, count: int, shape=None, device: str = "cpu", seed_offset: int = 0):
    """`count` tensors of the workload's value distribution, from one seeded stream.

    Values are drawn in fp32 and cast to bf16 with torch's own conversion when
    the workload is bf16.  Returns torch tensors on `device`.
    """
    import torch

    if shape is None:
        shape = (w.total_tokens, w.heads, w.head_dim)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed * 1000 + seed_offset)
    out = []
    for _ in range(count):
        if w.value_dist == "uniform_pm1":
            t = torch.rand(shape, generator=gen, device=device, dtype=torch.float32) * 2.0 - 1.0
        else:
            t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
            if w.value_std != 1.0:
                t.mul_(w.value_std)
        if w.dtype == "bf16":
            t = t.to(torch.bfloat16)
        out.append(t)
    return out


def scaled(w: Workload, total_tokens: Optional[int] = None, heads: Optional[int] = None,
           head_dim: Optional[int] = None) -> Workload:
    """Same distributions and seed at a smaller size (for oracle-sized parity runs)."""
    from dataclasses import replace

    return replace(w, total_tokens=total_tokens or w.total_tokens, heads=heads or w.heads,
                   head_dim=head_dim or w.head_dim,
                   name=f"{w.name}@T{total_tokens or w.total_tokens}")
