"""The unit-tile permutation kernels start their row lookups from the host's
record of the metadata (the shape it had when the host built it at that
address) and check the header before they load anything from the tensors; the
row-chunk kernel (records of packed-contiguous or one-document metadata; the
1 KiB bf16 rows and 2 KiB fp32 gradients here take it) loads its row under the
recorded shape and checks the header before it stores.  The layouts also run in
1.5 KiB rows, which take the unit tiles whatever the record.  A header whose shape
differs from the record (the buffer rewritten behind the host's back, here by a
device copy of other metadata) has the rows redone from the header.  Every such
case must still give the oracle's layout, inverse layout and gradient return
for the metadata the buffer now holds: record and header differing in policy,
in document count (one, across the staged-table limit), and in whether the row
maps are present."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, O, bits_equal, say, to_np

pytestmark = pytest.mark.gpu

T, W, H, D = 8192, 4, 4, 128


@pytest.fixture(scope="module")
def cp():
    from thd_token_layout_amd import cpthd
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return cpthd


def documents(kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "pc":  # 30 documents of random lengths
        cuts = np.sort(rng.choice(np.arange(1, T), size=29, replace=False))
        return np.concatenate([[0], cuts, [T]]).astype(np.int32)
    B = {"dcs1": 1, "dcs18": 18, "dcs116": 116}[kind]
    lengths = np.full(B, 2 * W, np.int64)  # every document at least one chunk per rank
    extra = rng.multinomial(T // (2 * W) - B, np.ones(B) / B)
    lengths += 2 * W * extra
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


POLICY = {"pc": O.PACKED_CONTIGUOUS, "dcs1": O.DUAL_CHUNK_SWAP, "dcs18": O.DUAL_CHUNK_SWAP,
          "dcs116": O.DUAL_CHUNK_SWAP}


def build(cp, kind, seed, row_maps, nbytes=None):
    cu = documents(kind, seed)
    code = cp.CP_POLICY_PACKED_CONTIGUOUS if kind == "pc" else cp.CP_POLICY_DUAL_CHUNK_SWAP
    buf = torch.empty(nbytes, dtype=torch.uint8, device=DEV) if nbytes else None
    meta = cp.cp_build_meta(torch.from_numpy(cu).to(DEV), T, W, code, meta=buf, check=True, row_maps=row_maps)
    return meta, cu


def rewritten(cp, rec_kind, rec_maps, now_kind, now_maps):
    """Metadata of `now_kind` copied on the device into a buffer the host recorded
    as `rec_kind`; returns a Meta over that buffer and the cu it now holds.  The
    recorded buffer is large enough for both (the kernels read the tables the
    header describes): 96 KiB, or 8 KiB for dual-chunk-swap without row maps
    (a buffer below the maps' size, so none are built)."""
    maps_bytes = cp.cp_meta_bytes_row_maps(116, W, T)
    assert 8 << 10 < cp.cp_meta_bytes_row_maps(1, W, T) and maps_bytes <= 96 << 10
    rec_bytes = (8 << 10) if rec_kind != "pc" and not rec_maps else (96 << 10)
    rec, _ = build(cp, rec_kind, 1, rec_maps, rec_bytes)
    assert bool(cp.read_row_maps(rec)) == rec_maps if rec_kind != "pc" else True
    now, cu = build(cp, now_kind, 2, now_maps)
    assert now.buf.numel() <= rec.buf.numel()
    rec.buf[: now.buf.numel()].copy_(now.buf)
    torch.cuda.synchronize()
    stale = cp.Meta(rec.buf, now.cp_size, now.policy, now.num_docs, now.total_tokens)
    return stale, cu, now


CASES = [("dcs116", True, "pc", False), ("dcs116", True, "dcs18", False), ("dcs116", True, "dcs1", True),
         ("pc", False, "dcs18", False), ("pc", False, "dcs116", True), ("dcs18", False, "dcs116", False),
         ("dcs18", False, "pc", False), ("dcs1", True, "dcs116", False), ("dcs1", False, "pc", False),
         ("pc", False, "dcs1", False)]


@pytest.mark.parametrize("rec_kind,rec_maps,now_kind,now_maps", CASES)
def test_layout_follows_the_header(cp, rec_kind, rec_maps, now_kind, now_maps):
    say(f"case stale record {rec_kind}{'+maps' if rec_maps else ''} -> header {now_kind}"
        f"{'+maps' if now_maps else ''}")
    stale, cu, _ = rewritten(cp, rec_kind, rec_maps, now_kind, now_maps)
    gen = torch.Generator(device=DEV).manual_seed(7)
    for h in (H, 6):  # 1 KiB rows (the record decides the kernel), 1.5 KiB rows (never row chunks)
        x = torch.randn((T, h, D), generator=gen, device=DEV).to(torch.bfloat16)
        parts = cp.cp_partition_thd(x, stale)
        back = cp.cp_gather_thd(parts, stale)
        assert cp.cp_meta_status(stale)[0] == cp.CP_OK
        ref = O.partition(to_np(x), cu, W, POLICY[now_kind])
        assert bits_equal(to_np(parts), ref), h
        assert bits_equal(to_np(back), to_np(x)), h


@pytest.mark.parametrize("rec_kind,rec_maps,now_kind,now_maps", CASES)
def test_grad_return_follows_the_header(cp, rec_kind, rec_maps, now_kind, now_maps):
    say(f"case stale record grad {rec_kind}{'+maps' if rec_maps else ''} -> header {now_kind}"
        f"{'+maps' if now_maps else ''}")
    stale, cu, _ = rewritten(cp, rec_kind, rec_maps, now_kind, now_maps)
    gen = torch.Generator(device=DEV).manual_seed(8)
    grads = [[torch.randn((T, H, D), generator=gen, device=DEV) for _ in range(W)]]
    slots = [[[torch.empty((T // W, H, D), device=DEV) for _ in range(W)] for _ in range(W)]]
    out = [[torch.empty((T // W, H, D), device=DEV) for _ in range(W)]]
    cp.cp_grad_return(grads, slots, out, stale)
    assert cp.cp_meta_status(stale)[0] == cp.CP_OK
    ref_slots, ref_out = O.grad_return([to_np(g) for g in grads[0]], cu, W, "f32", "f32",
                                       policy=POLICY[now_kind])
    for o in range(W):
        for w in range(W):
            assert bits_equal(to_np(slots[0][o][w]), ref_slots[o][w]), (o, w)
        assert bits_equal(to_np(out[0][o]), ref_out[o]), o


@pytest.mark.parametrize("rec_kind,rec_maps", [("pc", False), ("dcs1", True), ("dcs1", False), ("dcs116", True),
                                               ("dcs18", False)])
def test_rewritten_for_another_token_count_writes_nothing(cp, rec_kind, rec_maps):
    """The buffer rewritten with metadata of another token count (T/2) while the host's
    record still says T: every kernel loads under the record's shape (inside the tensors and
    the recorded metadata extent), then the header check fails, so nothing is stored and the
    call records a token-count mismatch; the row chunks (pc, dcs1 records) and the unit tiles
    (dcs116, dcs18) alike."""
    say(f"case stale record {rec_kind}{'+maps' if rec_maps else ''} -> header for T/2")
    rec_bytes = (8 << 10) if rec_kind != "pc" and not rec_maps else (96 << 10)
    rec, _ = build(cp, rec_kind, 3, rec_maps, rec_bytes)
    half = cp.cp_build_meta(torch.tensor([0, T // 2], dtype=torch.int32, device=DEV), T // 2, W,
                            cp.CP_POLICY_DUAL_CHUNK_SWAP, check=True, row_maps=False)
    assert half.buf.numel() <= rec.buf.numel()
    rec.buf[: half.buf.numel()].copy_(half.buf)
    torch.cuda.synchronize()
    gen = torch.Generator(device=DEV).manual_seed(9)
    x = torch.randn((T, H, D), generator=gen, device=DEV).to(torch.bfloat16)
    parts = torch.full((W, T // W, H, D), 5.0, dtype=torch.bfloat16, device=DEV)
    back = torch.full_like(x, 5.0)
    cp.cp_partition_thd(x, rec, parts=parts)
    cp.cp_gather_thd(x.view(W, T // W, H, D), rec, x=back)
    grads = [[torch.randn((T, H, D), generator=gen, device=DEV) for _ in range(W)]]
    slots = [[[torch.full((T // W, H, D), 5.0, device=DEV) for _ in range(W)] for _ in range(W)]]
    out = [[torch.full((T // W, H, D), 5.0, device=DEV) for _ in range(W)]]
    cp.cp_grad_return(grads, slots, out, rec)
    st, flags, _ = cp.cp_meta_status(rec)
    assert st == cp.CP_ERR_META and flags & cp.CP_CALL_TOKENS_MISMATCH, (st, flags)
    assert (parts == 5.0).all() and (back == 5.0).all()
    for o in range(W):
        assert (out[0][o] == 5.0).all()
        for w in range(W):
            assert (slots[0][o][w] == 5.0).all()
