"""The seeded input recipe: document-length distributions, shapes, value
distributions and determinism of the synthetic workloads (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import cp_oracle as O
from thd_token_layout_amd import workloads as WL


@pytest.mark.parametrize("name", ["dcs_t32k_w4", "dcs_s256k_w4"])
def test_loguniform_documents(name):
    w = WL.WORKLOADS[name]
    lengths = WL.doc_lengths(w.doc_lengths, w.total_tokens, w.seed)
    assert sum(lengths) == w.total_tokens
    assert all(L % 8 == 0 and L > 0 for L in lengths)             # multiples of 8 (2W for W = 4)
    assert all(256 <= L <= 8192 for L in lengths[:-1])            # only the last one is truncated
    assert lengths[-1] <= 8192
    # log-uniform on [256, 8192]: the median length is near sqrt(256 * 8192) ~ 1448
    assert 700 < np.median(lengths) < 3000
    cu = WL.cu_seqlens(w)
    assert O.cu_violations(cu, w.total_tokens, w.cp_size, O.DUAL_CHUNK_SWAP) == set()


@pytest.mark.parametrize("name", ["pc_t64k_w4", "pc_s256k_w4"])
def test_uniform_documents(name):
    w = WL.WORKLOADS[name]
    lengths = WL.doc_lengths(w.doc_lengths, w.total_tokens, w.seed)
    assert sum(lengths) == w.total_tokens
    assert all(1 <= L <= 4096 for L in lengths)
    # most documents are not divisible by 2W, the reason packed-contiguous exists
    assert np.mean([L % (2 * w.cp_size) != 0 for L in lengths]) > 0.6
    cu = WL.cu_seqlens(w)
    assert O.cu_violations(cu, w.total_tokens, w.cp_size, O.PACKED_CONTIGUOUS) == set()
    assert O.cu_violations(cu, w.total_tokens, w.cp_size, O.DUAL_CHUNK_SWAP) != set()


def test_fixed_and_single_documents():
    assert WL.cu_seqlens(WL.WORKLOADS["tiny_w2"]).tolist() == [0, 8, 24, 48]
    for name in ("grad_s256k_w4", "fused_s128k_w8", "dcs1_s256k_w4"):
        w = WL.WORKLOADS[name]
        assert WL.cu_seqlens(w).tolist() == [0, w.total_tokens]


def test_shapes_of_the_pages_workloads():
    g = WL.WORKLOADS["grad_s256k_w4"]
    assert (g.cp_size, g.total_tokens, g.heads, g.head_dim, g.dtype) == (4, 262144, 20, 128, "f32")
    f = WL.WORKLOADS["fused_s128k_w8"]
    assert (f.cp_size, f.total_tokens, f.heads, f.head_dim, f.dtype, f.out_dtype) == \
        (8, 131072, 32, 128, "bf16", "bf16")
    assert WL.SWEEP_BYTES == [1024 * 2 ** k for k in range(15)] and WL.SWEEP_BYTES[-1] == 16 << 20


def test_values_are_seeded_and_distributed_as_stated():
    w = WL.scaled(WL.WORKLOADS["grad_s256k_w4"], total_tokens=2048)
    a = WL.random_tensors(w, 2)
    b = WL.random_tensors(w, 2)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    assert not torch.equal(a[0], a[1])
    v = a[0].double()
    assert abs(v.mean().item()) < 1e-5 and abs(v.std().item() - 1e-3) < 2e-5
    t = WL.random_tensors(WL.WORKLOADS["tiny_w2"], 1)[0]
    assert t.dtype == torch.float32 and t.min() >= -1.0 and t.max() < 1.0
    q = WL.random_tensors(WL.scaled(WL.WORKLOADS["dcs_t32k_w4"], total_tokens=1024), 1)[0]
    assert q.dtype == torch.bfloat16 and abs(q.float().std().item() - 1.0) < 0.02
