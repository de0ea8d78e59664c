"""GPU parity of the row-chunk permutation kernel, which serves metadata whose row map
has a closed form (packed-contiguous, and dual-chunk-swap with one document) when rows
are a multiple of 1 KiB: one wave per 1 KiB of a written row, the row's source and
destination from the ownership formula.  Partition, gather and gradient scatter against
the oracle element by element, for row lengths of 1, 2, 5 and 10 KiB, W = 1, 2, 3, 4 and
8, the degenerate shapes (n = T/W = 1 or 2, so a chunk of one row under dual-chunk-swap),
several tensors in one call, tensors not 256-byte aligned, and a check of which kernel each
call launched (rows of 1.5 KiB and metadata of two documents, with or without row maps,
keep the unit tiles)."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, O, bits_equal, say, to_np

pytestmark = pytest.mark.gpu

PC, DCS = "packed_contiguous", "dual_chunk_swap"


@pytest.fixture(scope="module")
def cp():
    from thd_token_layout_amd import cpthd
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return cpthd


def launched(cp, fn):
    cp.cp_profile_enable(True)
    fn()
    prof = cp.cp_profile_read()
    cp.cp_profile_enable(False)
    return [k for k in prof if k.startswith("permute")]


def meta_for(cp, cu, T, W, policy, row_maps=True):
    return cp.cp_build_meta(torch.from_numpy(np.asarray(cu, np.int32)).to(DEV), T, W, cp.POLICY[policy],
                            check=True, row_maps=row_maps)


# (T, W, policy, H, D, dtype): rows of H * D * size bytes
LAYOUT_CASES = [
    (4104, 4, DCS, 4, 128, torch.bfloat16),    # 1 KiB rows, n = 1026, c = 513
    (4104, 4, PC, 8, 128, torch.bfloat16),     # 2 KiB
    (6000, 3, DCS, 20, 128, torch.bfloat16),   # 5 KiB, W = 3
    (6000, 3, PC, 20, 128, torch.float32),     # 10 KiB
    (4096, 8, DCS, 2, 128, torch.float32),     # 1 KiB, W = 8
    (999, 1, PC, 4, 128, torch.bfloat16),      # one rank, odd T
    (1000, 1, DCS, 8, 64, torch.float32),      # one rank: two chunks of 500 rows
    (8, 4, DCS, 4, 128, torch.bfloat16),       # n = 2: chunks of one row
    (4, 4, PC, 4, 128, torch.bfloat16),        # n = 1
    (16, 8, PC, 2, 256, torch.bfloat16),       # n = 2, W = 8
]


@pytest.mark.parametrize("T,W,policy,H,D,dt", LAYOUT_CASES)
def test_layouts(cp, T, W, policy, H, D, dt):
    say(f"case row chunks layout T={T} W={W} {policy} [{H},{D}] {dt}")
    cu = np.array([0, T], np.int32)
    meta = meta_for(cp, cu, T, W, policy)
    gen = torch.Generator(device=DEV).manual_seed(T + W)
    x = torch.randn((T, H, D), generator=gen, device=DEV).to(dt)
    parts = torch.empty((W, T // W, H, D), dtype=dt, device=DEV)
    back = torch.empty_like(x)
    names = launched(cp, lambda: cp.cp_partition_thd(x, meta, parts=parts))
    names += launched(cp, lambda: cp.cp_gather_thd(parts, meta, x=back))
    assert names == ["permute_chunk<1KiB>", "permute_chunk<1KiB,g>"], names
    assert cp.cp_meta_status(meta)[0] == cp.CP_OK
    ref = O.partition(to_np(x), cu, W, policy)
    assert bits_equal(to_np(parts), ref)
    assert bits_equal(to_np(back), to_np(x))
    # the gather of other parts (not the partition's own output) against the oracle
    other = torch.randn((W, T // W, H, D), generator=gen, device=DEV).to(dt)
    cp.cp_gather_thd(other, meta, x=back)
    assert bits_equal(to_np(back), O.gather(to_np(other), cu, W, policy))


@pytest.mark.parametrize("policy", [PC, DCS])
def test_several_tensors_one_launch(cp, policy):
    """Three small tensors in one call: one launch with a tensor per grid row."""
    T, W = 2048, 4
    say(f"case row chunks multi {policy}")
    cu = np.array([0, T], np.int32)
    meta = meta_for(cp, cu, T, W, policy)
    gen = torch.Generator(device=DEV).manual_seed(5)
    xs = [torch.randn((T, 8, 128), generator=gen, device=DEV).to(torch.bfloat16) for _ in range(3)]
    parts = [torch.empty((W, T // W, 8, 128), dtype=torch.bfloat16, device=DEV) for _ in xs]
    backs = [torch.empty_like(x) for x in xs]
    assert launched(cp, lambda: cp.cp_partition_thd_multi(xs, meta, parts=parts)) == ["permute_chunk<1KiB>"]
    assert launched(cp, lambda: cp.cp_gather_thd_multi(parts, meta, xs=backs)) == ["permute_chunk<1KiB,g>"]
    for x, p, b in zip(xs, parts, backs):
        assert bits_equal(to_np(p), O.partition(to_np(x), cu, W, policy))
        assert bits_equal(to_np(b), to_np(x))


SCATTER_CASES = [(4104, 4, DCS, 4, 128, torch.float32), (4104, 4, PC, 4, 128, torch.float32),
                 (6000, 3, DCS, 20, 128, torch.float32), (4096, 8, PC, 4, 128, torch.bfloat16),
                 (8, 4, DCS, 8, 128, torch.float32), (2048, 2, DCS, 8, 128, torch.bfloat16)]


@pytest.mark.parametrize("T,W,policy,H,D,dt", SCATTER_CASES)
def test_grad_scatter(cp, T, W, policy, H, D, dt):
    """The gradient return's scatter through the row chunks (each writer's rows into its
    slot of every owner): every slot and owner sum against the oracle."""
    say(f"case row chunks scatter T={T} W={W} {policy} [{H},{D}] {dt}")
    cu = np.array([0, T], np.int32)
    meta = meta_for(cp, cu, T, W, policy)
    gen = torch.Generator(device=DEV).manual_seed(T * W)
    grads = [[(torch.randn((T, H, D), generator=gen, device=DEV) * 1e-2).to(dt) for _ in range(W)]]
    n = T // W
    slots = [[[torch.empty((n, H, D), dtype=dt, device=DEV) for _ in range(W)] for _ in range(W)]]
    out = [[torch.empty((n, H, D), dtype=dt, device=DEV) for _ in range(W)]]
    names = launched(cp, lambda: cp.cp_grad_return(grads, slots, out, meta))
    assert names == ["permute_chunk<1KiB,owners>"], names
    assert cp.cp_meta_status(meta)[0] == cp.CP_OK
    tag = "f32" if dt == torch.float32 else "bf16"
    ref_slots, ref_out = O.grad_return([to_np(g) for g in grads[0]], cu, W, tag, tag, policy=policy)
    for o in range(W):
        for w in range(W):
            assert bits_equal(to_np(slots[0][o][w]), ref_slots[o][w]), (o, w)
        assert bits_equal(to_np(out[0][o]), ref_out[o]), o


@pytest.mark.parametrize("what", ["rows of 1.5 KiB", "two documents", "two documents, no row maps", "no record"])
def test_other_shapes_keep_unit_tiles(cp, what):
    """Rows not a multiple of 1 KiB, or a row map that needs the row maps or the document
    tables, take the unit tiles; metadata the host has no record of takes the row tiles.
    Results against the oracle either way."""
    T, W = 4096, 4
    say(f"case row chunks not taken: {what}")
    H, cu = (6, [0, T]) if what == "rows of 1.5 KiB" else (4, [0, 1024, T])
    meta = meta_for(cp, cu, T, W, DCS, row_maps=what != "two documents, no row maps")
    if what == "no record":
        # a copy at an address no buffer of the allocator starts at (272 bytes into a new
        # allocation), so no metadata was ever built there
        nb = meta.buf.numel()
        view = torch.empty(nb + 1024, dtype=torch.uint8, device=DEV)[272: 272 + nb]
        view.copy_(meta.buf)
        meta = cp.Meta(view, meta.cp_size, meta.policy, meta.num_docs, meta.total_tokens)
    gen = torch.Generator(device=DEV).manual_seed(9)
    x = torch.randn((T, H, 128), generator=gen, device=DEV).to(torch.bfloat16)
    parts = torch.empty((W, T // W, H, 128), dtype=torch.bfloat16, device=DEV)
    names = launched(cp, lambda: cp.cp_partition_thd(x, meta, parts=parts))
    want = "permute_rows" if what == "no record" else "permute_flat"
    assert len(names) == 1 and names[0].startswith(want), names
    assert bits_equal(to_np(parts), O.partition(to_np(x), np.array(cu, np.int32), W, DCS))


@pytest.mark.parametrize("policy", [PC, DCS])
@pytest.mark.parametrize("offset", [16, 48, 1040])
def test_unaligned_to_the_chunk(cp, policy, offset):
    """Tensors that start 16, 48 or 1040 bytes into an allocation (16-byte aligned, so the
    row chunks still serve them, but neither 256-byte nor 1 KiB aligned), rows of 1 KiB (fp16
    layouts, bf16 gradients): layouts and gradient scatter against the oracle, bytes around
    the layout outputs untouched."""
    T, W, H, D = 1032, 4, 4, 128
    say(f"case row chunks at byte offset {offset} {policy}")
    cu = np.array([0, T], np.int32)
    meta = meta_for(cp, cu, T, W, policy)
    rb = H * D * 2
    gen = torch.Generator(device=DEV).manual_seed(offset)

    def view(shape, fill=None, dt=torch.float16):
        n = int(np.prod(shape)) * 2
        raw = torch.empty(n + offset + 1024, dtype=torch.uint8, device=DEV)
        if fill is None:
            raw.copy_(torch.randint(0, 256, raw.shape, generator=gen, device=DEV, dtype=torch.int64).to(torch.uint8))
        else:
            raw.fill_(fill)
        return raw, raw[offset: offset + n].view(dt).view(shape)

    _, x = view((T, H, D))
    x.copy_(torch.randn((T, H, D), generator=gen, device=DEV).to(torch.float16))
    raw_p, parts = view((W, T // W, H, D), fill=0xA5)
    raw_b, back = view((T, H, D), fill=0x5A)
    names = launched(cp, lambda: cp.cp_partition_thd(x, meta, parts=parts))
    names += launched(cp, lambda: cp.cp_gather_thd(parts, meta, x=back))
    assert names == ["permute_chunk<1KiB>", "permute_chunk<1KiB,g>"], names
    assert bits_equal(to_np(parts), O.partition(to_np(x), cu, W, policy))
    assert bits_equal(to_np(back), to_np(x))
    for raw, n in ((raw_p, parts.numel() * 2), (raw_b, back.numel() * 2)):
        fill = 0xA5 if raw is raw_p else 0x5A
        assert (raw[:offset] == fill).all() and (raw[offset + n:] == fill).all()
    assert rb == 1024
    bf = torch.bfloat16
    grads = [[view((T, H, D), dt=bf)[1] for _ in range(W)]]
    for g in grads[0]:
        g.copy_(torch.randn((T, H, D), generator=gen, device=DEV).to(bf))
    slots = [[[view((T // W, H, D), dt=bf)[1] for _ in range(W)] for _ in range(W)]]
    out = [[view((T // W, H, D), dt=bf)[1] for _ in range(W)]]
    assert launched(cp, lambda: cp.cp_grad_return(grads, slots, out, meta)) == ["permute_chunk<1KiB,owners>"]
    ref_slots, ref_out = O.grad_return([to_np(g) for g in grads[0]], cu, W, "bf16", "bf16", policy=policy)
    for o in range(W):
        for w in range(W):
            assert bits_equal(to_np(slots[0][o][w]), ref_slots[o][w]), (o, w)
        assert bits_equal(to_np(out[0][o]), ref_out[o]), o
