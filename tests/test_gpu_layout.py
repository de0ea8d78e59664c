"""GPU parity of the metadata builder, THD partition and inverse gather against the
CPU oracle: bit-exact, on the tiny hand-worked case, the packed-document
workloads at full size, the S=262144 shapes (full compare of one tensor plus
round trips), and edge cases (empty input and documents, W=1 and W=64, ragged
and unaligned rows, invalid and mismatched metadata)."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import DEV, O, WL, bits_equal, policy_name, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cp():
    from thd_token_layout_amd import cpthd
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return cpthd


def build(cp, cu_np, T, W, policy, check=True, row_maps=True):
    cu = torch.from_numpy(np.asarray(cu_np, dtype=np.int32)).to(DEV)
    return cp.cp_build_meta(cu, T, W, policy, check=check, row_maps=row_maps)


def check_meta_against_oracle(cp, meta, cu_np, T, W, pol):
    local, n_local = cp.read_local_cu(meta)
    ref_local, ref_n = O.local_cu_seqlens(np.asarray(cu_np), T, W, pol)
    assert bits_equal(local.numpy(), ref_local), (local, ref_local)
    assert bits_equal(n_local.numpy(), ref_n), (n_local, ref_n)


def check_layout(cp, x, cu_np, W, pol_code, full=True, sample_rows=4096, seed=0, row_maps=True):
    """partition vs oracle, gather vs oracle, round trip; returns parts."""
    T = x.shape[0]
    pol = policy_name(pol_code)
    meta = build(cp, cu_np, T, W, pol_code, row_maps=row_maps)
    check_meta_against_oracle(cp, meta, cu_np, T, W, pol)
    parts = cp.cp_partition_thd(x, meta)
    back = cp.cp_gather_thd(parts, meta)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16) if x.dtype != torch.float32 else back.view(torch.int32),
                       x.view(torch.int16) if x.dtype != torch.float32 else x.view(torch.int32))
    xn = to_np(x)
    if full:
        ref = O.partition(xn, np.asarray(cu_np), W, pol)
        assert bits_equal(to_np(parts), ref)
        ref_back = O.gather(ref, np.asarray(cu_np), W, pol)
        assert bits_equal(to_np(back), ref_back)
    else:
        rng = np.random.default_rng(seed)
        n = T // W
        for r in range(W):
            rows = O.rank_rows(np.asarray(cu_np), T, W, pol, r)
            idx = np.unique(np.concatenate([rng.integers(0, n, size=sample_rows), [0, n - 1]]))
            got = to_np(parts[r][torch.from_numpy(idx).to(DEV)])
            assert bits_equal(got, xn[rows[idx]]), (r,)
    meta_status = cp.cp_meta_status(meta)
    assert meta_status[0] == cp.CP_OK, meta_status
    return parts


# ------------------------------------------------------------------ tiny hand-worked case
def test_tiny_dcs_and_pc(cp):
    w = WL.WORKLOADS["tiny_w2"]
    say("case tiny_w2")
    cu = WL.cu_seqlens(w)
    (x,) = WL.random_tensors(w, 1)
    x = x.to(DEV)
    for W in (1, 2, 4):
        check_layout(cp, x, cu, W, cp.CP_POLICY_DUAL_CHUNK_SWAP)
        check_layout(cp, x, cu, W, cp.CP_POLICY_PACKED_CONTIGUOUS)
    check_layout(cp, x, cu, 3, cp.CP_POLICY_PACKED_CONTIGUOUS)
    # the hand-worked ownership table, through the GPU: x[t] = t
    xi = torch.arange(48, dtype=torch.float32, device=DEV)[:, None, None].expand(48, 2, 8).contiguous()
    g = __import__("pins").golden()
    for W in (2, 4):
        parts = cp.cp_partition_thd(xi, build(cp, cu, 48, W, cp.CP_POLICY_DUAL_CHUNK_SWAP))
        got = parts[:, :, 0, 0].cpu().numpy().astype(int).tolist()
        assert got == g["dual_chunk_swap"][str(W)]["rows"]


@pytest.mark.parametrize("row_maps", [True, False])
@pytest.mark.parametrize("name", ["dcs_t32k_w4", "pc_t64k_w4"])
def test_packed_documents_full_size(cp, name, row_maps):
    """Without the row maps the 18-document dual-chunk-swap workload stages its document
    tables in LDS; with them it looks rows up in the maps."""
    w = WL.WORKLOADS[name]
    say(f"case {name} row maps {row_maps}")
    cu = WL.cu_seqlens(w)
    pol = cp.POLICY[w.policy]
    for x in WL.random_tensors(w, w.n_tensors, device=DEV):  # Q, K, V
        check_layout(cp, x, cu, w.cp_size, pol, row_maps=row_maps)


@pytest.mark.parametrize("name", ["dcs_t32k_w4", "pc_t64k_w4"])
def test_multi_tensor_calls(cp, name):
    """Q, K, V in one launch: every tensor equals the oracle's partition, the
    gather restores each, and outputs overlapping each other are rejected."""
    w = WL.WORKLOADS[name]
    say(f"case {name} multi-tensor")
    cu = WL.cu_seqlens(w)
    pol = cp.POLICY[w.policy]
    xs = WL.random_tensors(w, w.n_tensors, device=DEV)
    meta = build(cp, cu, w.total_tokens, w.cp_size, pol)
    parts = cp.cp_partition_thd_multi(xs, meta)
    backs = cp.cp_gather_thd_multi(parts, meta)
    for x, p, b in zip(xs, parts, backs):
        assert bits_equal(to_np(p), O.partition(to_np(x), cu, w.cp_size, policy_name(pol)))
        assert bits_equal(to_np(b), to_np(x))
    big = torch.empty((2 * w.total_tokens, w.heads, w.head_dim), dtype=xs[0].dtype, device=DEV)
    shaped = (w.cp_size, w.total_tokens // w.cp_size, w.heads, w.head_dim)
    overlapping = [big[: w.total_tokens].view(shaped), big[w.total_tokens // 2: 3 * w.total_tokens // 2].view(shaped),
                   parts[2]]
    with pytest.raises(cp.CpError) as e:
        cp.cp_partition_thd_multi(xs, meta, parts=overlapping)
    assert e.value.status == cp.CP_ERR_ALIAS


@pytest.mark.parametrize("name", ["dcs_s256k_w4", "pc_s256k_w4", "dcs1_s256k_w4"])
def test_s256k_shapes(cp, name):
    w = WL.WORKLOADS[name]
    say(f"case {name}")
    cu = WL.cu_seqlens(w)
    pol = cp.POLICY[w.policy]
    xs = WL.random_tensors(w, w.n_tensors, device=DEV)
    for k, x in enumerate(xs):
        check_layout(cp, x, cu, w.cp_size, pol, full=(k == 0), seed=k)
        torch.cuda.empty_cache()


# ------------------------------------------------------------------ edge cases
def test_empty_input(cp):
    say("case empty")
    for pol in (0, 1):
        cu = torch.zeros(1, dtype=torch.int32, device=DEV)
        meta = cp.cp_build_meta(cu, 0, 4, pol, check=True)
        x = torch.empty((0, 2, 8), dtype=torch.bfloat16, device=DEV)
        parts = cp.cp_partition_thd(x, meta)
        assert parts.shape == (4, 0, 2, 8)
        back = cp.cp_gather_thd(parts, meta)
        assert back.shape == (0, 2, 8)
        local, n_local = cp.read_local_cu(meta)
        assert (local == 0).all() and (n_local == 0).all()


@pytest.mark.parametrize("W,lengths", [(2, [0, 4, 0, 8, 0]), (4, [8, 0, 0, 16, 8]),
                                       (3, [0, 6, 12, 0])])
def test_empty_documents_dcs(cp, W, lengths):
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    x = torch.randn((T, 3, 16), device=DEV)
    check_layout(cp, x, cu, W, cp.CP_POLICY_DUAL_CHUNK_SWAP)


@pytest.mark.parametrize("W,lengths", [(2, [0, 5, 0, 7, 0]), (4, [3, 0, 0, 13, 0]),
                                       (8, [1, 2, 3, 4, 5, 6, 7, 4]), (5, [25])])
def test_empty_and_odd_documents_pc(cp, W, lengths):
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    x = torch.randn((T, 2, 8), device=DEV)
    check_layout(cp, x, cu, W, cp.CP_POLICY_PACKED_CONTIGUOUS)


def test_w64_and_many_documents(cp):
    say("case W=64")
    rng = np.random.default_rng(11)
    W = 64
    lengths = (rng.integers(0, 4, size=40) * 2 * W).tolist()
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    x = torch.randn((T, 1, 64), device=DEV).to(torch.bfloat16)
    check_layout(cp, x, cu, W, cp.CP_POLICY_DUAL_CHUNK_SWAP)
    check_layout(cp, x, cu, W, cp.CP_POLICY_PACKED_CONTIGUOUS)
    # many documents: B large relative to the block size of the metadata builder
    lengths = (rng.integers(1, 3, size=3000) * 8).tolist()
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    x = torch.randn((T, 2, 8), device=DEV)
    check_layout(cp, x, cu, 4, cp.CP_POLICY_DUAL_CHUNK_SWAP)
    check_layout(cp, x, cu, 4, cp.CP_POLICY_PACKED_CONTIGUOUS)


@pytest.mark.parametrize("row_maps", [False, True])
@pytest.mark.parametrize("B,H,D,dtype", [(4100, 2, 8, torch.float32),      # 64 B rows: 4 rows per wave
                                         (40000, 1, 16, torch.float32),    # 64 B rows, 40000 documents
                                         (4500, 20, 128, torch.bfloat16),  # 5 KiB rows (the Q,K,V shape)
                                         (4000, 20, 128, torch.float32)])  # 10 KiB rows: 2 waves per row
def test_thousands_of_documents(cp, B, H, D, dtype, row_maps):
    """Dual-chunk-swap metadata of more than 63^2 = 3969 documents (empty ones among them),
    with and without the row maps: without them the row tiles' wave search over the document
    table takes three rounds of 64 probes (below that one or two); with them the unit tiles
    look rows up in the maps (rows of at least ~1 KiB).  Every element of partition and gather
    against the oracle."""
    say(f"case {B} documents [{H},{D}] {dtype} row maps {row_maps}")
    rng = np.random.default_rng(B + H)
    lengths = rng.integers(0, 4, size=B) * 8
    lengths[0] = max(int(lengths[0]), 8)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    x = torch.randn((T, H, D), device=DEV).to(dtype)
    check_layout(cp, x, cu, 4, cp.CP_POLICY_DUAL_CHUNK_SWAP, row_maps=row_maps)


@pytest.mark.parametrize("B,W,T", [(65, 4, 65 * 8 * 3), (200, 8, 200 * 16 * 2), (3000, 2, 3000 * 4 * 5),
                                   (66, 64, 66 * 128)])
def test_row_maps_equal_the_oracle_map(cp, B, W, T):
    """The row maps cp_build_meta writes (dual-chunk-swap, a buffer of cp_meta_bytes_row_maps
    bytes) hold exactly the oracle's ownership map: row_of_local[r n + i] is the global row of
    rank r's local row i, local_of_row its inverse.  A buffer of cp_meta_bytes only, or
    packed-contiguous metadata, gives no maps (header field 0)."""
    say(f"case row maps B={B} W={W} T={T}")
    rng = np.random.default_rng(B * W)
    lengths = rng.multinomial(T // (2 * W) - B, np.ones(B) / B) * 2 * W + 2 * W
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    assert cu[-1] == T
    pol = cp.CP_POLICY_DUAL_CHUNK_SWAP
    meta = build(cp, cu, T, W, pol)
    assert meta.buf.numel() >= cp.cp_meta_bytes_row_maps(B, W, T)
    l2g, g2l = cp.read_row_maps(meta)
    ref = O.partition(np.arange(T, dtype=np.int64)[:, None], cu, W, policy_name(pol)).reshape(-1)
    assert (l2g.numpy() == ref).all()
    inv = np.empty(T, dtype=np.int64)
    inv[ref] = np.arange(T)
    assert (g2l.numpy() == inv).all()
    # one document: the maps of Megatron's native layout
    one = build(cp, np.array([0, T], dtype=np.int32), T, W, pol)
    l2g1, _ = cp.read_row_maps(one)
    ref1 = O.partition(np.arange(T, dtype=np.int64)[:, None], np.array([0, T]), W, policy_name(pol)).reshape(-1)
    assert (l2g1.numpy() == ref1).all()
    # no maps: a buffer of the tables alone, or packed-contiguous metadata
    small = build(cp, cu, T, W, pol, row_maps=False)
    assert cp.read_row_maps(small) is None
    pc = build(cp, cu, T, W, cp.CP_POLICY_PACKED_CONTIGUOUS)
    assert cp.read_row_maps(pc) is None


@pytest.mark.parametrize("H,D,dtype", [(3, 5, torch.bfloat16),     # 30 B rows: 2-byte units
                                       (1, 6, torch.float32),      # 24 B rows: 8-byte units
                                       (3, 3, torch.float32),      # 36 B rows: 4-byte units
                                       (8, 136, torch.bfloat16),   # 2176 B: ragged lane tail
                                       (40, 128, torch.float32),   # 20 KiB rows: several passes
                                       (1, 8, torch.float16)])
def test_ragged_rows(cp, H, D, dtype):
    cu = np.array([0, 16, 24, 64, 64, 128], dtype=np.int32)
    x = torch.randn((128, H, D), device=DEV).to(dtype)
    check_layout(cp, x, cu, 4, cp.CP_POLICY_DUAL_CHUNK_SWAP)
    check_layout(cp, x, cu, 4, cp.CP_POLICY_PACKED_CONTIGUOUS)


def test_unaligned_base_pointers(cp):
    cu = np.array([0, 32, 64], dtype=np.int32)
    flat = torch.randn(64 * 2 * 8 + 1, device=DEV).to(torch.bfloat16)
    x = flat[1:].view(64, 2, 8)  # data_ptr is 2 bytes past a 256-byte boundary
    assert x.data_ptr() % 16 == 2
    out_flat = torch.zeros(64 * 2 * 8 + 3, device=DEV, dtype=torch.bfloat16)
    parts = out_flat[3:].view(4, 16, 2, 8)
    meta = build(cp, cu, 64, 4, cp.CP_POLICY_DUAL_CHUNK_SWAP)
    cp.cp_partition_thd(x, meta, parts=parts)
    ref = O.partition(to_np(x), cu, 4, O.DUAL_CHUNK_SWAP)
    assert bits_equal(to_np(parts), ref)
    back_flat = torch.zeros(64 * 2 * 8 + 5, device=DEV, dtype=torch.bfloat16)
    back = back_flat[5:].view(64, 2, 8)
    cp.cp_gather_thd(parts, meta, x=back)
    assert bits_equal(to_np(back), to_np(x))


def test_more_tiles_than_the_grid(cp):
    """68M rows of 16 bytes: more row tiles than the largest grid launched, so the
    kernels' grid-stride loops run; checked by round trip on the device and by
    sampled rows against the oracle's one-row map."""
    say("case 68M rows (grid-stride)")
    lengths = [1 << 26, (1 << 20) + 4, 12]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    W = 2
    x = torch.randint(-2**15, 2**15, (T, 2, 4), dtype=torch.int16, device=DEV).view(torch.bfloat16)
    rng = np.random.default_rng(5)
    for pol in (cp.CP_POLICY_DUAL_CHUNK_SWAP, cp.CP_POLICY_PACKED_CONTIGUOUS):
        meta = build(cp, cu, T, W, pol)
        parts = cp.cp_partition_thd(x, meta)
        back = cp.cp_gather_thd(parts, meta)
        torch.cuda.synchronize()
        assert torch.equal(back.view(torch.int16), x.view(torch.int16))
        n = T // W
        for r in range(W):
            idx = np.unique(np.concatenate([rng.integers(0, n, size=300), [0, n - 1, n - 7]]))
            g = [O.rank_row(cu, T, W, policy_name(pol), r, int(i)) for i in idx]
            got = to_np(parts[r][torch.from_numpy(idx).to(DEV)])
            assert bits_equal(got, to_np(x[torch.tensor(g, device=DEV)])), (pol, r)
        del parts, back
    torch.cuda.empty_cache()


@pytest.mark.parametrize("pol,lengths", [
    (1, [7, 0, 93, 20]), (1, [120]),          # packed-contiguous: 8 KiB unit tiles
    (0, [120]), (0, [8]),                     # one document: 12 KiB unit tiles
    (0, [16, 0, 8, 0, 40, 8, 0, 24]),         # a few documents: 12 KiB unit tiles
    (0, [8, 0, 16] * 13),                     # 39 documents: unit tiles, tables staged in LDS
    (0, [8] * 65),                            # more than 64 documents: row tiles
])
@pytest.mark.parametrize("units", [55, 65, 100, 333, 1280])
def test_unit_tiles_ragged(cp, pol, lengths, units):
    """Rows of 16-byte units whose count does not divide the unit tile, so tiles
    start and end inside rows and the last tile is partial; one tensor and three
    tensors per call; every output against the oracle."""
    W = 4
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    say(f"case unit tiles pol={pol} T={T} row={16 * units} B")
    gen = torch.Generator(device=DEV).manual_seed(units + T)
    xs = [torch.randint(-2**15, 2**15, (T, 1, 8 * units), dtype=torch.int16, device=DEV,
                        generator=gen).view(torch.bfloat16) for _ in range(3)]
    check_layout(cp, xs[0], cu, W, pol)
    meta = build(cp, cu, T, W, pol)
    parts = cp.cp_partition_thd_multi(xs, meta)
    backs = cp.cp_gather_thd_multi(parts, meta)
    for x, p, bk in zip(xs, parts, backs):
        assert bits_equal(to_np(p), O.partition(to_np(x), cu, W, policy_name(pol)))
        assert bits_equal(to_np(bk), to_np(x))


def test_buffers_smaller_than_the_sizes_are_rejected(cp):
    """A call whose sizes run past the end of a buffer's allocation is refused on the
    host (CP_ERR_SHAPE) before anything is launched."""
    say("case buffers past their allocation")
    torch.cuda.empty_cache()
    x = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    parts = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    meta = build(cp, np.array([0, 64], dtype=np.int32), 64, 4, cp.CP_POLICY_DUAL_CHUNK_SWAP)
    T = (1 << 31) - 8  # 2^31 rows of 512 bytes: 1 TiB, more than the device holds
    st = cp.lib.cp_partition_thd(x.data_ptr(), parts.data_ptr(), T, 1, 256, cp.CP_BF16, meta.ptr(), None)
    assert st == cp.CP_ERR_SHAPE
    st = cp.lib.cp_slot_sum(2, (ctypes.c_void_p * 2)(x.data_ptr(), parts.data_ptr()), parts.data_ptr(),
                            1 << 38, cp.CP_F32, cp.CP_F32, 0, None)
    assert st == cp.CP_ERR_SHAPE
    grads = (ctypes.c_void_p * 2)(x.data_ptr(), x.data_ptr())
    outs = (ctypes.c_void_p * 2)(parts.data_ptr(), parts.data_ptr())
    st = cp.lib.cp_grad_return_fused(-1, 2, 1, grads, outs, T - 2040, 1, 256, cp.CP_F32, cp.CP_F32,
                                     meta.ptr(), 0, None)
    assert st == cp.CP_ERR_SHAPE
    torch.cuda.synchronize()
    assert (x == 0).all() and (parts == 0).all()  # nothing was launched


def test_extent_check_inside_one_allocation(cp):
    """Buffers of one call that lie in one allocation are checked against that
    allocation's end even when the runtime is asked about it only once: a slot
    that starts 256 bytes before the end and runs 512 bytes is refused.  The
    allocation is made with hipMalloc directly, so its extent is exactly known
    (through the library's own handle: the HIP runtime this process already uses)."""
    say("case extent of a second buffer in the same allocation")
    hip = ctypes.CDLL(cp.LIB_PATH)
    hip.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    hip.hipMemset.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t]
    hip.hipFree.argtypes = [ctypes.c_void_p]
    size = 64 << 20
    base = ctypes.c_void_p()
    assert hip.hipMalloc(ctypes.byref(base), size) == 0
    try:
        assert hip.hipMemset(base, 0, size) == 0
        out = torch.zeros(128, dtype=torch.float32, device=DEV)
        end = base.value + size
        slots = (ctypes.c_void_p * 2)(base.value, end - 256)
        assert cp.lib.cp_slot_sum(2, slots, out.data_ptr(), 128, cp.CP_F32, cp.CP_F32, 0, None) == cp.CP_ERR_SHAPE
        slots = (ctypes.c_void_p * 2)(base.value, end - 512)  # ends exactly at the allocation's end
        assert cp.lib.cp_slot_sum(2, slots, out.data_ptr(), 128, cp.CP_F32, cp.CP_F32, 0, None) == cp.CP_OK
        torch.cuda.synchronize()
        assert (out == 0).all()
    finally:
        torch.cuda.synchronize()
        hip.hipFree(base)


def test_stale_host_record_changes_no_result(cp):
    """The host's record of a metadata buffer only picks the tile shape.  Overwrite a
    buffer built for 3 documents with metadata of 100 documents (a plain device copy,
    which the host does not see): the unit-tile kernel then finds more documents than
    it can stage and searches the metadata itself; the result still equals the oracle."""
    say("case stale host record")
    W, T = 4, 800
    cu_small = np.array([0, 200, 200, 800], dtype=np.int32)
    cu_big = np.arange(0, T + 1, 8, dtype=np.int32)  # 100 documents of 8 tokens
    x = torch.randint(-2**15, 2**15, (T, 1, 520), dtype=torch.int16, device=DEV).view(torch.bfloat16)
    for pol in (cp.CP_POLICY_DUAL_CHUNK_SWAP, cp.CP_POLICY_PACKED_CONTIGUOUS):
        big = build(cp, cu_big, T, W, pol)
        buf = torch.zeros(big.buf.numel(), dtype=torch.uint8, device=DEV)
        small = cp.cp_build_meta(torch.from_numpy(cu_small).to(DEV), T, W, cp.CP_POLICY_DUAL_CHUNK_SWAP,
                                 meta=buf, check=True)
        buf.copy_(big.buf)  # the record still says: dual-chunk-swap, 3 documents
        stale = cp.Meta(buf, W, pol, len(cu_big) - 1, T)
        parts = cp.cp_partition_thd(x, stale)
        back = cp.cp_gather_thd(parts, stale)
        assert bits_equal(to_np(parts), O.partition(to_np(x), cu_big, W, policy_name(pol))), pol
        assert bits_equal(to_np(back), to_np(x)), pol
        assert cp.cp_meta_status(stale)[0] == cp.CP_OK
        del small


def test_unit_tiles_more_than_the_grid(cp):
    """2^31 + 4096 units of 16 bytes (32 GiB per buffer) under packed-contiguous
    metadata: more unit tiles than the largest grid launched, so the unit-tile
    kernel's grid-stride loop runs.  Rows hold their own index, so every sampled
    row of the partition and of the gather is checked against the oracle's map."""
    T, W, words = (1 << 25) + 64, 4, 128  # rows of 1 KiB = 128 int64 words
    say(f"case unit tiles beyond the grid: T={T}, 1 KiB rows")
    x = torch.empty((T, 1, 512), dtype=torch.bfloat16, device=DEV)
    torch.add(torch.arange(T, dtype=torch.int64, device=DEV)[:, None] * words,
              torch.arange(words, dtype=torch.int64, device=DEV)[None, :], out=x.view(torch.int64).view(T, words))
    cu = np.array([0, 1000, T], dtype=np.int32)
    meta = build(cp, cu, T, W, cp.CP_POLICY_PACKED_CONTIGUOUS)
    parts = cp.cp_partition_thd(x, meta)
    x.zero_()
    cp.cp_gather_thd(parts, meta, x=x)
    n = T // W
    rng = np.random.default_rng(11)
    cols = np.arange(words, dtype=np.int64)
    for r in range(W):
        idx = np.unique(np.concatenate([rng.integers(0, n, size=200), [0, n - 1]]))
        got = parts[r][torch.from_numpy(idx).to(DEV)].view(torch.int64).view(-1, words).cpu().numpy()
        g = np.array([O.rank_row(cu, T, W, O.PACKED_CONTIGUOUS, r, int(i)) for i in idx], dtype=np.int64)
        assert (got == g[:, None] * words + cols[None, :]).all(), r
    idx = np.unique(np.concatenate([rng.integers(0, T, size=800), [0, T - 1]]))
    got = x[torch.from_numpy(idx).to(DEV)].view(torch.int64).view(-1, words).cpu().numpy()
    assert (got == idx[:, None].astype(np.int64) * words + cols[None, :]).all()
    assert cp.cp_meta_status(meta)[0] == cp.CP_OK
    del x, parts
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ invalid / mismatched metadata
FLAG_NAMES = {"first_not_zero": 0x1, "decreasing": 0x2, "last_not_total": 0x4,
              "doc_not_divisible": 0x8}


@pytest.mark.parametrize("cu,T,W,pol", [
    ([0, 8, 24, 48], 48, 8, 0),           # 8 % 16 != 0 (hand-worked rejection)
    ([1, 8, 48], 48, 1, 1),
    ([0, 30, 24, 48], 48, 2, 1),
    ([0, 8, 24, 40], 48, 2, 0),
    ([2, 30, 20, 40], 48, 2, 0),
])
def test_invalid_cu_is_flagged_and_nothing_written(cp, cu, T, W, pol):
    meta = build(cp, cu, T, W, pol, check=False)
    st, flags, _ = cp.cp_meta_status(meta)
    want = 0
    for name in O.cu_violations(cu, T, W, policy_name(pol)):
        want |= FLAG_NAMES[name]
    assert st == cp.CP_ERR_META and (flags & cp.CP_META_BUILD_MASK) == want, (hex(flags), want)
    x = torch.randn((T, 2, 8), device=DEV)
    parts = torch.full((T,), 7.0, device=DEV).view(W, T // W, 1, 1).expand(W, T // W, 2, 8).contiguous() \
        if T % W == 0 else None
    if parts is not None:
        before = parts.clone()
        cp.cp_partition_thd(x, meta, parts=parts)
        torch.cuda.synchronize()
        assert torch.equal(parts, before)
        st, flags, _ = cp.cp_meta_status(meta)
        assert flags & cp.CP_CALL_USED_INVALID_META


def test_meta_mismatch_and_host_errors(cp):
    cu = np.array([0, 16, 32], dtype=np.int32)
    meta = build(cp, cu, 32, 2, cp.CP_POLICY_DUAL_CHUNK_SWAP)
    x = torch.randn((48, 2, 8), device=DEV)  # 48 tokens, meta says 32
    parts = torch.zeros((2, 24, 2, 8), device=DEV)
    cp.cp_partition_thd(x, meta, parts=parts)
    st, flags, _ = cp.cp_meta_status(meta)
    assert st == cp.CP_ERR_META and flags & cp.CP_CALL_TOKENS_MISMATCH
    assert torch.count_nonzero(parts) == 0
    # host pointer -> CP_ERR_DEVICE; overlapping output -> CP_ERR_ALIAS; FP8 -> unsupported
    meta = build(cp, cu, 32, 2, cp.CP_POLICY_DUAL_CHUNK_SWAP)
    xh = torch.randn((32, 2, 8))
    with pytest.raises(cp.CpError) as e:
        cp.cp_partition_thd(xh, meta, parts=torch.zeros((2, 16, 2, 8), device=DEV))
    assert e.value.status == cp.CP_ERR_DEVICE
    buf = torch.randn((64, 2, 8), device=DEV)
    with pytest.raises(cp.CpError) as e:
        cp.cp_partition_thd(buf[:32], meta, parts=buf[16:48].view(2, 16, 2, 8))
    assert e.value.status == cp.CP_ERR_ALIAS
    if hasattr(torch, "float8_e4m3fn"):
        x8 = torch.zeros((32, 2, 8), device=DEV).to(torch.float8_e4m3fn)
        with pytest.raises(cp.CpError) as e:
            cp.cp_partition_thd(x8, meta, parts=torch.zeros((2, 16, 2, 8), device=DEV).to(torch.float8_e4m3fn))
        assert e.value.status == cp.CP_ERR_UNSUPPORTED
    with pytest.raises(cp.CpError) as e:
        cp.cp_build_meta(torch.tensor([0, 5, 10], dtype=torch.int32, device=DEV), 10, 4, 1)
    assert e.value.status == cp.CP_ERR_SHAPE


# ------------------------------------------------------------------ largest token count
def test_largest_token_count(cp):
    """T = 2^31 - 8 tokens (the largest multiple of 2W = 8 the ABI accepts), rows of
    16 bytes holding their own index: partition and gather under both policies,
    the attention-step tables, every index kept in 64 bits where it must be.
    Sampled rows against the oracle's one-row map."""
    T, W = (1 << 31) - 8, 4
    say(f"case largest token count T={T}")
    x = torch.empty((T, 1, 2), dtype=torch.int64, device=DEV)
    x[:, 0, 0] = torch.arange(T, dtype=torch.int64, device=DEV)
    x[:, 0, 1] = -x[:, 0, 0]
    xf = x.view(torch.float32).view(T, 1, 4)  # 16-byte rows
    rng = np.random.default_rng(31)
    n = T // W
    for pol, cu in ((cp.CP_POLICY_DUAL_CHUNK_SWAP, np.array([0, T], dtype=np.int32)),
                    (cp.CP_POLICY_PACKED_CONTIGUOUS, np.array([0, 1000, T - 8, T], dtype=np.int32))):
        meta = build(cp, cu, T, W, pol)
        parts = cp.cp_partition_thd(xf, meta)
        for r in range(W):
            idx = np.unique(np.concatenate([rng.integers(0, n, size=200), [0, n - 1]]))
            got = parts[r][torch.from_numpy(idx).to(DEV)].view(torch.int64).view(-1, 2).cpu().numpy()
            g = np.array([O.rank_row(cu, T, W, policy_name(pol), r, int(i)) for i in idx], dtype=np.int64)
            assert (got[:, 0] == g).all() and (got[:, 1] == -g).all(), (pol, r)
        back = torch.zeros_like(xf)
        cp.cp_gather_thd(parts, meta, x=back)
        del parts
        idx = np.unique(np.concatenate([rng.integers(0, T, size=500), [0, T - 1]]))
        got = back[torch.from_numpy(idx).to(DEV)].view(torch.int64).view(-1, 2).cpu().numpy()
        assert (got[:, 0] == idx).all() and (got[:, 1] == -idx).all(), pol
        del back
        magic, tables = cp.read_attn_meta(cp.cp_build_attn_meta(meta), len(cu) - 1, W)
        assert magic == cp.CP_ATTN_MAGIC
        for k, v in O.attention_meta(cu, T, W, policy_name(pol)).items():
            assert np.array_equal(tables[k].numpy(), v), (pol, k)
        assert cp.cp_meta_status(meta)[0] == cp.CP_OK
        torch.cuda.empty_cache()
    del x, xf
    torch.cuda.empty_cache()
