"""Randomized GPU parity: seeded random configurations (CP size, policy, document
lengths with empty documents, row shapes including unaligned ones, dtypes,
tensor counts, accumulate mode) run through every entry point of the C ABI and
compared bit-exactly with the CPU oracle.  Each case prints its parameters
before it runs."""
import os

import numpy as np
import pytest
import torch

from gpu_util import DEV, O, bits_equal, say, to_np

pytestmark = pytest.mark.gpu

POL = {0: O.DUAL_CHUNK_SWAP, 1: O.PACKED_CONTIGUOUS}
TAG = {torch.float32: "f32", torch.bfloat16: "bf16"}
ROWS = [(1, 1), (1, 3), (2, 8), (3, 5), (1, 64), (4, 32), (8, 17), (2, 128), (1, 520), (5, 128)]
# 160 cases by default; CPTHD_RANDOM_CASES raises the count for a longer run.
N_CASES = int(os.environ.get("CPTHD_RANDOM_CASES", "160"))


@pytest.fixture(scope="module")
def cp():
    from thd_token_layout_amd import cpthd
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return cpthd


def random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    W = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    pol = int(rng.integers(0, 2))
    B = int(rng.integers(1, 40))
    if pol == 0:
        lengths = rng.integers(0, 6, size=B) * 2 * W
        if lengths.sum() == 0:
            lengths[-1] = 2 * W
    else:
        lengths = rng.integers(0, 60, size=B)
        lengths[rng.random(B) < 0.2] = 0
        lengths[-1] += (-int(lengths.sum())) % W + W
    H, D = ROWS[int(rng.integers(0, len(ROWS)))]
    if int(lengths.sum()) * H * D * W * W > 1 << 25:  # keep the host-side oracle work small
        H, D = 2, 8
    return rng, W, pol, np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32), H, D


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_case(cp, seed):
    rng, W, pol, cu, H, D = random_case(seed)
    T = int(cu[-1])
    B = len(cu) - 1
    layout_dt = [torch.float32, torch.bfloat16, torch.float16][int(rng.integers(0, 3))]
    in_dt, out_dt = [(torch.float32, torch.float32), (torch.float32, torch.bfloat16),
                     (torch.bfloat16, torch.bfloat16), (torch.bfloat16, torch.float32)][int(rng.integers(0, 4))]
    n_t = int(rng.integers(1, 4))
    accumulate = bool(rng.integers(0, 2))
    row_maps = seed % 2 == 0  # half the cases build the dual-chunk-swap row maps
    say(f"case random seed={seed}: W={W} policy={pol} B={B} T={T} row=[{H},{D}] layout={layout_dt} "
        f"grad {in_dt}->{out_dt} tensors={n_t} accumulate={accumulate} row maps={row_maps}")
    gen = torch.Generator(device=DEV).manual_seed(seed)
    meta = cp.cp_build_meta(torch.from_numpy(cu).to(DEV), T, W, pol, check=True, row_maps=row_maps)

    # metadata and attention-step tables
    local, n_local = cp.read_local_cu(meta)
    ref_local, ref_n = O.local_cu_seqlens(cu, T, W, POL[pol])
    assert bits_equal(local.numpy(), ref_local) and bits_equal(n_local.numpy(), ref_n)
    magic, tables = cp.read_attn_meta(cp.cp_build_attn_meta(meta), B, W)
    assert magic == cp.CP_ATTN_MAGIC
    for k, v in O.attention_meta(cu, T, W, POL[pol]).items():
        assert np.array_equal(tables[k].numpy(), v), k

    # partition / gather of n_t tensors in one call
    xs = [torch.randn((T, H, D), generator=gen, device=DEV).to(layout_dt) for _ in range(n_t)]
    parts = cp.cp_partition_thd_multi(xs, meta)
    backs = cp.cp_gather_thd_multi(parts, meta)
    for x, p, bk in zip(xs, parts, backs):
        assert bits_equal(to_np(p), O.partition(to_np(x), cu, W, POL[pol]))
        assert bits_equal(to_np(bk), to_np(x))

    # gradient return, unfused and fused, optionally accumulating
    n = T // W
    grads = [[(torch.randn((T, H, D), generator=gen, device=DEV) * 1e-3).to(in_dt) for _ in range(W)]
             for _ in range(2)]
    into = [[(torch.randn((n, H, D), generator=gen, device=DEV) * 1e-3).to(out_dt) for _ in range(W)]
            for _ in range(2)]
    slots = [[[torch.empty((n, H, D), dtype=in_dt, device=DEV) for _ in range(W)] for _ in range(W)]
             for _ in range(2)]
    out = [[v.clone() for v in row] for row in into]
    fused = [[v.clone() for v in row] for row in into]
    epochs = torch.zeros((W, W), dtype=torch.int32, device=DEV)
    cp.cp_grad_return(grads, slots, out, meta, epochs=epochs, epoch=seed + 1, accumulate=accumulate)
    cp.cp_grad_return_fused(grads, fused, meta, accumulate=accumulate)
    st = cp.cp_meta_status(meta)
    assert st[0] == cp.CP_OK, st
    assert (epochs == seed + 1).all()
    for t in range(2):
        gn = [to_np(g) for g in grads[t]]
        iv = [to_np(v) for v in into[t]] if accumulate else None
        ref_slots, ref_out = O.grad_return(gn, cu, W, TAG[in_dt], TAG[out_dt], policy=POL[pol], into=iv)
        for o in range(W):
            for w in range(W):
                assert bits_equal(to_np(slots[t][o][w]), ref_slots[o][w]), (t, o, w)
            assert bits_equal(to_np(out[t][o]), ref_out[o]), (t, o)
            assert bits_equal(to_np(fused[t][o]), ref_out[o]), (t, o)
