"""Every document split of small token counts through the GPU path: metadata,
attention-step tables, partition and gather, each bit-exact against the oracle
(packed-contiguous: T <= 8; dual-chunk-swap: up to 4 chunk-lengths per rank;
W = 1..4), the layouts in rows of 64 bytes (row tiles) and of 1 KiB (row chunks for
packed-contiguous and one-document metadata, unit tiles with row maps otherwise)."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, O, bits_equal, say, to_np

pytestmark = pytest.mark.gpu
POL = {0: O.DUAL_CHUNK_SWAP, 1: O.PACKED_CONTIGUOUS}


def compositions(total):
    if total == 0:
        yield []
        return
    for first in range(1, total + 1):
        for rest in compositions(total - first):
            yield [first] + rest


def cases():
    for W in (1, 2, 3, 4):
        for T in range(0, 9):
            if T % W == 0:
                for lengths in compositions(T):
                    yield W, 1, lengths
        for units in range(0, 5):
            for chunks in compositions(units):
                yield W, 0, [2 * W * c for c in chunks]


@pytest.fixture(scope="module")
def cp():
    from thd_token_layout_amd import cpthd
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return cpthd


@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_every_small_document_split(cp, W):
    n_cases = 0
    for w, pol, lengths in cases():
        if w != W:
            continue
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        T, B = int(cu[-1]), len(lengths)
        tag = f"W={W} policy={pol} lengths={lengths}"
        meta = cp.cp_build_meta(torch.from_numpy(cu).to(DEV), T, W, pol, check=True)
        local, n_local = cp.read_local_cu(meta)
        ref_local, ref_n = O.local_cu_seqlens(cu, T, W, POL[pol])
        assert bits_equal(local.numpy(), ref_local) and bits_equal(n_local.numpy(), ref_n), tag
        magic, tab = cp.read_attn_meta(cp.cp_build_attn_meta(meta), B, W)
        assert magic == cp.CP_ATTN_MAGIC, tag
        for k, v in O.attention_meta(cu, T, W, POL[pol]).items():
            assert np.array_equal(tab[k].numpy(), v), (tag, k)
        if T:
            x = torch.arange(T * 16, dtype=torch.float32, device=DEV).reshape(T, 2, 8)
            parts = cp.cp_partition_thd(x, meta)
            assert bits_equal(to_np(parts), O.partition(to_np(x), cu, W, POL[pol])), tag
            assert bits_equal(to_np(cp.cp_gather_thd(parts, meta)), to_np(x)), tag
            # 1 KiB rows: the row chunks (packed-contiguous, one document) and the unit tiles
            # with row maps (several documents)
            y = torch.arange(T * 256, dtype=torch.float32, device=DEV).reshape(T, 2, 128)
            py = cp.cp_partition_thd(y, meta)
            assert bits_equal(to_np(py), O.partition(to_np(y), cu, W, POL[pol])), tag
            assert bits_equal(to_np(cp.cp_gather_thd(py, meta)), to_np(y)), tag
        n_cases += 1
    say(f"case exhaustive small splits W={W}: {n_cases} splits")
    assert n_cases > 10
