"""GPU parity of the owner gradient return (scatter, epochs, fixed-order slot sum),
the fused scatter+sum and the small-message slot sum against the CPU oracle:
bit-exact at oracle-sized shapes, sampled rows plus fused == unfused at the full
S=262144 / S=131072 shapes, order and sign pins, per-rank protocol mode on
separate streams with a delayed writer and NaN-poisoned slots, and the
host-forced epoch timeout."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, O, WL, bits_equal, say, to_np

pytestmark = pytest.mark.gpu

TAG = {torch.float32: "f32", torch.bfloat16: "bf16"}


@pytest.fixture(scope="module")
def cp():
    from thd_token_layout_amd import cpthd
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return cpthd


def make_meta(cp, cu_np, T, W, row_maps=True):
    cu = torch.from_numpy(np.asarray(cu_np, dtype=np.int32)).to(DEV)
    return cp.cp_build_meta(cu, T, W, cp.CP_POLICY_DUAL_CHUNK_SWAP, check=True, row_maps=row_maps)


def alloc(grads, W, out_dtype, fill=None):
    n_t = len(grads)
    T, H, D = grads[0][0].shape
    n = T // W
    mk = (lambda dt: torch.full((n, H, D), fill, dtype=dt, device=DEV)) if fill is not None else \
        (lambda dt: torch.empty((n, H, D), dtype=dt, device=DEV))
    slots = [[[mk(grads[0][0].dtype) for _ in range(W)] for _ in range(W)] for _ in range(n_t)]
    out = [[mk(out_dtype) for _ in range(W)] for _ in range(n_t)]
    return slots, out


def oracle_full(grads, cu, W, out_tag):
    """Oracle results for every tensor: (slots[t][o][w], out[t][o])."""
    res = []
    for gt in grads:
        gn = [to_np(g) for g in gt]
        res.append(O.grad_return(gn, np.asarray(cu), W, TAG[gt[0].dtype], out_tag))
    return res


def run_and_check_full(cp, grads, cu, W, out_dtype, epochs=None, epoch=0):
    T = grads[0][0].shape[0]
    meta = make_meta(cp, cu, T, W)
    slots, out = alloc(grads, W, out_dtype)
    cp.cp_grad_return(grads, slots, out, meta, epochs=epochs, epoch=epoch)
    fused = [[torch.empty_like(o) for o in row] for row in out]
    cp.cp_grad_return_fused(grads, fused, meta)
    st = cp.cp_meta_status(meta)
    assert st[0] == cp.CP_OK, st
    ref = oracle_full(grads, cu, W, TAG[out_dtype])
    for t in range(len(grads)):
        ref_slots, ref_out = ref[t]
        for o in range(W):
            for w in range(W):
                assert bits_equal(to_np(slots[t][o][w]), ref_slots[o][w]), (t, o, w)
            assert bits_equal(to_np(out[t][o]), ref_out[o]), (t, o)
            assert bits_equal(to_np(fused[t][o]), ref_out[o]), (t, o)
    return meta


# ------------------------------------------------------------------ tiny case (C1)
def test_tiny_grad_return(cp):
    w = WL.WORKLOADS["tiny_w2"]
    say("case tiny_w2 grad return")
    cu = WL.cu_seqlens(w)
    vals = WL.random_tensors(w, 4, device=DEV)  # writers 0,1 x {dK, dV}
    grads = [[vals[0], vals[1]], [vals[2], vals[3]]]
    epochs = torch.zeros((2, 2), dtype=torch.int32, device=DEV)
    run_and_check_full(cp, grads, cu, 2, torch.float32, epochs=epochs, epoch=5)
    assert (epochs.cpu().numpy().view(np.uint32) == O.epochs_after(2, 5)).all()
    # exact-integer pin through the GPU: G_w[t] = (w+1)(t+1)
    t = torch.arange(48, dtype=torch.float32, device=DEV)[:, None, None]
    gi = [[((wr + 1) * (t + 1)).expand(48, 2, 8).contiguous() for wr in range(2)]]
    meta = make_meta(cp, cu, 48, 2)
    slots, out = alloc(gi, 2, torch.float32)
    cp.cp_grad_return(gi, slots, out, meta)
    g = __import__("pins").golden()["integer_grad_return_w2"]
    assert out[0][0][:5, 0, 0].cpu().tolist() == g["owner0_first"]
    assert out[0][1][:5, 0, 0].cpu().tolist() == g["owner1_first"]


@pytest.mark.parametrize("W,in_dt,out_dt", [
    (2, torch.float32, torch.float32), (3, torch.float32, torch.float32),
    (4, torch.float32, torch.float32), (4, torch.bfloat16, torch.bfloat16),
    (4, torch.bfloat16, torch.float32), (8, torch.bfloat16, torch.bfloat16),
    (8, torch.float32, torch.float32), (12, torch.float32, torch.float32),
    (16, torch.bfloat16, torch.bfloat16)])
def test_random_documents(cp, W, in_dt, out_dt):
    say(f"case random docs W={W} {in_dt}->{out_dt}")
    rng = np.random.default_rng(W)
    lengths = (rng.integers(0, 6, size=7) * 2 * W).tolist()
    lengths[-1] += 2 * W * 4
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    gen = torch.Generator(device=DEV).manual_seed(W)
    grads = [[(torch.randn((T, 3, 40), generator=gen, device=DEV) * 1e-3).to(in_dt) for _ in range(W)]
             for _ in range(2)]
    run_and_check_full(cp, grads, cu, W, out_dt)


@pytest.mark.parametrize("policy", ["dual_chunk_swap", "packed_contiguous"])
@pytest.mark.parametrize("T", [56, 200])
def test_unit_tiles_straddling_owners(cp, policy, T):
    """The scatter's unit tiles write each tile through one buffer resource when its rows lie
    in one owner's slot, and row by row when the tile straddles two owners: with 1.5 KiB rows a
    tile covers 8 rows, so T/W = 14 or 50 rows per owner puts owner boundaries inside tiles.
    The unit-tile kernel is the one launched (checked; rows of 1.5 KiB, not a multiple of
    1 KiB, keep packed-contiguous metadata off the row chunks), every slot and output
    against the oracle."""
    W, H, D = 4, 3, 128
    say(f"case straddling tiles {policy} T={T}")
    cu = np.array([0, 24, T], dtype=np.int32)  # two documents, each a multiple of 2W
    gen = torch.Generator(device=DEV)
    gen.manual_seed(T)
    grads = [[torch.randn((T, H, D), device=DEV, generator=gen) for _ in range(W)]]
    pol = cp.POLICY[policy]
    meta = cp.cp_build_meta(torch.from_numpy(cu).to(DEV), T, W, pol, check=True)
    slots, out = alloc(grads, W, torch.float32)
    cp.cp_profile_enable(True)
    cp.cp_grad_return(grads, slots, out, meta)
    prof = cp.cp_profile_read()
    cp.cp_profile_enable(False)
    assert any(k.startswith("permute_flat") for k in prof), prof
    ref_slots, ref_out = O.grad_return([to_np(g) for g in grads[0]], cu, W, "f32", "f32", policy=policy)
    for o in range(W):
        for w in range(W):
            assert bits_equal(to_np(slots[0][o][w]), ref_slots[o][w]), (o, w)
        assert bits_equal(to_np(out[0][o]), ref_out[o]), o


def test_profile_select_records_one_kernel(cp):
    """cp_profile_select limits the launch timing to one kernel name; None restores all."""
    say("case profile select")
    T, W = 4096, 4
    cu = np.array([0, T], dtype=np.int32)
    gen = torch.Generator(device=DEV).manual_seed(11)
    grads = [[torch.randn((T, 4, 128), device=DEV, generator=gen) for _ in range(W)]]
    meta = make_meta(cp, cu, T, W)
    slots, out = alloc(grads, W, torch.float32)
    cp.cp_profile_enable(True)
    cp.cp_grad_return(grads, slots, out, meta)
    every = cp.cp_profile_read()
    scatter = next(k for k in every if k.startswith("permute"))
    assert any(k.startswith("slot_sum") for k in every), every
    cp.cp_profile_select(scatter)
    cp.cp_grad_return(grads, slots, out, meta)
    only = cp.cp_profile_read()
    cp.cp_profile_select(None)
    cp.cp_grad_return(grads, slots, out, meta)
    again = cp.cp_profile_read()
    cp.cp_profile_enable(False)
    assert list(only) == [scatter] and only[scatter][0] == W, only
    assert set(again) == set(every), (again, every)
    with pytest.raises(cp.CpError):
        cp.cp_profile_select("k" * 200)


@pytest.mark.parametrize("B,H,D", [(4100, 2, 64), (4000, 20, 128)])
def test_thousands_of_documents(cp, B, H, D):
    """The gradient return under dual-chunk-swap metadata of more than 3969 documents (a
    three-round wave search in the scatter's row tiles), 512-byte and 10 KiB fp32 rows:
    every slot, the unfused and the fused output against the oracle."""
    say(f"case grad return {B} documents [{H},{D}]")
    rng = np.random.default_rng(B + 7)
    lengths = rng.integers(0, 3, size=B) * 8
    lengths[0] = max(int(lengths[0]), 8)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    W = 4
    gen = torch.Generator(device=DEV)
    gen.manual_seed(B)
    grads = [[torch.randn((T, H, D), device=DEV, generator=gen) for _ in range(W)]]
    run_and_check_full(cp, grads, cu, W, torch.float32)


@pytest.mark.parametrize("W,H,D,in_dt,out_dt", [
    (4, 4, 128, torch.float32, torch.float32), (4, 8, 128, torch.float32, torch.bfloat16),
    (8, 4, 128, torch.bfloat16, torch.bfloat16), (4, 4, 128, torch.bfloat16, torch.float32),
    (2, 2, 256, torch.float32, torch.float32), (3, 12, 128, torch.float32, torch.float32),
    (4, 16, 128, torch.float32, torch.float32), (2, 20, 128, torch.float32, torch.bfloat16),
    (4, 16, 128, torch.bfloat16, torch.bfloat16), (3, 24, 128, torch.bfloat16, torch.float32)])
def test_vector_paths_full_compare(cp, W, H, D, in_dt, out_dt):
    """Rows of whole 512-element groups take the vectorized fused / slot-sum paths."""
    say(f"case vector paths W={W} [{H},{D}] {in_dt}->{out_dt}")
    rng = np.random.default_rng(100 + W)
    lengths = (rng.integers(1, 4, size=5) * 2 * W * 8).tolist()
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    gen = torch.Generator(device=DEV).manual_seed(W + H)
    grads = [[(torch.randn((T, H, D), generator=gen, device=DEV) * 1e-3).to(in_dt) for _ in range(W)]
             for _ in range(2)]
    run_and_check_full(cp, grads, cu, W, out_dt)


def test_order_and_negative_zero(cp):
    say("case order pin")
    cu = np.array([0, 64], dtype=np.int32)
    vals = [1e8, 1.0, -1e8, 1.0]
    grads = [[torch.full((64, 1, 8), v, device=DEV) for v in vals]]
    meta = make_meta(cp, cu, 64, 4)
    slots, out = alloc(grads, 4, torch.float32)
    cp.cp_grad_return(grads, slots, out, meta)
    fused = [[torch.empty_like(o) for o in out[0]]]
    cp.cp_grad_return_fused(grads, fused, meta)
    for o in range(4):
        assert (out[0][o] == 1.0).all() and (fused[0][o] == 1.0).all()
    ss = torch.empty(1000, device=DEV)
    cp.cp_slot_sum([torch.full((1000,), v, device=DEV) for v in vals], ss)
    assert (ss == 1.0).all()
    # -0.0 survives: the accumulator is seeded with slot 0
    nz = [[torch.full((64, 1, 8), -0.0, device=DEV) for _ in range(4)]]
    cp.cp_grad_return(nz, slots, out, meta)
    cp.cp_grad_return_fused(nz, fused, meta)
    for o in range(4):
        assert (out[0][o].view(torch.int32) == -2**31).all()
        assert (fused[0][o].view(torch.int32) == -2**31).all()


def test_bf16_rounding_specials(cp):
    """fp32 sums that land on bf16 ties, NaN, inf, denormals: device RNE == oracle RNE."""
    say("case bf16 specials")
    bits = np.array([0x3F808000, 0x3F818000, 0x3F80FFFF, 0x7F7FFFFF, 0x00008000, 0x00018000,
                     0x80008000, 0x7FC00001, 0xFFA00000, 0x7F800000, 0xFF800000, 0x00000001,
                     0x3F7FFFFF, 0x477FE000, 0xC77FE000, 0x7F7F8000], dtype=np.uint32)
    f = bits.view(np.float32)
    n = 1024
    s0 = np.resize(f, n).astype(np.float32)
    s1 = np.zeros(n, dtype=np.float32)  # x + 0 = x except -0
    slots = [torch.from_numpy(s0).to(DEV), torch.from_numpy(s1).to(DEV)]
    for out_dt, tag in ((torch.bfloat16, "bf16"), (torch.float32, "f32")):
        out = torch.empty(n, dtype=out_dt, device=DEV)
        cp.cp_slot_sum(slots, out)
        ref = O.slot_sum([s0, s1], "f32", tag)
        got = to_np(out)
        if tag == "f32":
            nan = np.isnan(ref)
            assert bits_equal(got[~nan], ref[~nan]) and np.isnan(got[nan]).all()
        else:
            assert bits_equal(got, ref)


@pytest.mark.parametrize("n,W,in_dt,out_dt,offset", [
    (1, 8, torch.float32, torch.float32, 0), (7, 3, torch.float32, torch.float32, 0),
    (1000003, 8, torch.float32, torch.float32, 0), (4099, 5, torch.bfloat16, torch.bfloat16, 0),
    (4099, 5, torch.bfloat16, torch.float32, 0), (777, 4, torch.float32, torch.float32, 1),
    (777, 4, torch.bfloat16, torch.bfloat16, 3), (65536, 64, torch.float32, torch.float32, 0)])
def test_slot_sum_tails_and_alignment(cp, n, W, in_dt, out_dt, offset):
    gen = torch.Generator(device=DEV).manual_seed(n + W)
    bufs = [torch.randn(n + offset, generator=gen, device=DEV).to(in_dt) for _ in range(W)]
    slots = [b[offset:] for b in bufs]
    outb = torch.empty(n + offset, dtype=out_dt, device=DEV)
    out = outb[offset:]
    cp.cp_slot_sum(slots, out)
    ref = O.slot_sum([to_np(s) for s in slots], TAG[in_dt], TAG[out_dt])
    assert bits_equal(to_np(out), ref)


def test_small_message_sweep(cp):
    """W=8 fp32 slots of 1 KiB .. 16 MiB summed into one (every size, full compare)."""
    w = WL.WORKLOADS["sweep_w8"]
    for nbytes in WL.SWEEP_BYTES:
        n = nbytes // 4
        slots = WL.random_tensors(w, 8, shape=(n,), device=DEV, seed_offset=nbytes)
        out = torch.empty(n, device=DEV)
        cp.cp_slot_sum(slots, out)
        ref = O.slot_sum([to_np(s) for s in slots], "f32", "f32")
        assert bits_equal(to_np(out), ref), nbytes


# ------------------------------------------------------------------ full-size shapes
def sampled_check(cp, grads, slots, out, cu, W, out_dtype, n_samples=256, seed=0):
    """Oracle map + oracle sum on sampled owner rows (full shapes are too big to copy whole)."""
    T = grads[0][0].shape[0]
    n = T // W
    rng = np.random.default_rng(seed)
    for t in range(len(grads)):
        for o in range(W):
            rows = O.rank_rows(np.asarray(cu), T, W, O.DUAL_CHUNK_SWAP, o)
            idx = np.unique(np.concatenate([rng.integers(0, n, size=n_samples), [0, n // 2 - 1,
                                                                                 n // 2, n - 1]]))
            gidx = torch.from_numpy(rows[idx]).to(DEV)
            lidx = torch.from_numpy(idx).to(DEV)
            src = [to_np(grads[t][w].index_select(0, gidx)) for w in range(W)]
            ref = O.slot_sum(src, TAG[grads[t][0].dtype], TAG[out_dtype])
            assert bits_equal(to_np(out[t][o].index_select(0, lidx)), ref), (t, o)
            if slots is not None:
                for w in range(W):
                    assert bits_equal(to_np(slots[t][o][w].index_select(0, lidx)), src[w]), (t, o, w)


@pytest.mark.parametrize("row_maps", [True, False])
def test_grad_return_s256k_w4(cp, row_maps):
    """Both lookups of the scatter's unit tiles: the row maps, and without them the
    document tables staged in LDS."""
    w = WL.WORKLOADS["grad_s256k_w4"]
    say(f"case grad_s256k_w4 (full size) row maps {row_maps}")
    cu = WL.cu_seqlens(w)
    W = w.cp_size
    vals = WL.random_tensors(w, 2 * W, device=DEV)
    grads = [vals[:W], vals[W:]]  # dK, dV of writers 0..3
    meta = make_meta(cp, cu, w.total_tokens, W, row_maps=row_maps)
    slots, out = alloc(grads, W, torch.float32)
    epochs = torch.zeros((W, W), dtype=torch.int32, device=DEV)
    cp.cp_grad_return(grads, slots, out, meta, epochs=epochs, epoch=1)
    assert cp.cp_meta_status(meta)[0] == cp.CP_OK
    sampled_check(cp, grads, slots, out, cu, W, torch.float32)
    del slots
    torch.cuda.empty_cache()
    fused = [[torch.empty_like(o) for o in row] for row in out]
    cp.cp_grad_return_fused(grads, fused, meta)
    torch.cuda.synchronize()
    for t in range(2):
        for o in range(W):
            assert torch.equal(fused[t][o].view(torch.int32), out[t][o].view(torch.int32)), (t, o)
    assert (epochs == 1).all()


def test_fused_more_rows_than_the_grid(cp):
    """68M output rows of 4 fp32 (scalar fused path, one row per wave): more than the
    largest grid launched, so the grid-stride loop runs; sampled rows vs the oracle."""
    say("case fused 68M rows (grid-stride)")
    W = 2
    lengths = [1 << 26, (1 << 20) + 4, 12]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    gen = torch.Generator(device=DEV).manual_seed(68)
    grads = [[torch.randn((T, 1, 4), generator=gen, device=DEV) for _ in range(W)]]
    meta = make_meta(cp, cu, T, W)
    n = T // W
    out = [[torch.empty((n, 1, 4), device=DEV) for _ in range(W)]]
    cp.cp_grad_return_fused(grads, out, meta)
    rng = np.random.default_rng(6)
    for o in range(W):
        idx = np.unique(np.concatenate([rng.integers(0, n, size=300), [0, n - 1]]))
        g = torch.tensor([O.rank_row(cu, T, W, O.DUAL_CHUNK_SWAP, o, int(i)) for i in idx], device=DEV)
        src = [to_np(grads[0][w].index_select(0, g)) for w in range(W)]
        ref = O.slot_sum(src, "f32", "f32")
        assert bits_equal(to_np(out[0][o].index_select(0, torch.from_numpy(idx).to(DEV))), ref), o
    del grads, out
    torch.cuda.empty_cache()


def test_fused_s128k_w8(cp):
    w = WL.WORKLOADS["fused_s128k_w8"]
    say("case fused_s128k_w8 (full size)")
    cu = WL.cu_seqlens(w)
    W = w.cp_size
    vals = WL.random_tensors(w, 2 * W, device=DEV)
    grads = [vals[:W], vals[W:]]
    meta = make_meta(cp, cu, w.total_tokens, W)
    n = w.total_tokens // W
    fused = [[torch.empty((n, w.heads, w.head_dim), dtype=torch.bfloat16, device=DEV) for _ in range(W)]
             for _ in range(2)]
    cp.cp_grad_return_fused(grads, fused, meta)
    sampled_check(cp, grads, None, fused, cu, W, torch.bfloat16)
    slots, out = alloc(grads, W, torch.bfloat16)
    cp.cp_grad_return(grads, slots, out, meta)
    torch.cuda.synchronize()
    for t in range(2):
        for o in range(W):
            assert torch.equal(fused[t][o].view(torch.int16), out[t][o].view(torch.int16)), (t, o)


# ------------------------------------------------------------------ per-rank protocol mode
def per_rank_case(cp, W, seed):
    rng = np.random.default_rng(seed)
    lengths = (rng.integers(1, 5, size=5) * 2 * W * 16).tolist()
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    gen = torch.Generator(device=DEV).manual_seed(seed)
    grads = [[torch.randn((T, 4, 64), generator=gen, device=DEV) for _ in range(W)] for _ in range(2)]
    meta = make_meta(cp, cu, T, W)
    slots, out = alloc(grads, W, torch.float32, fill=float("nan"))
    epochs = torch.zeros((W, W), dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    return cu, grads, meta, slots, out, epochs


def check_per_rank_result(cp, meta, cu, grads, out, epochs, W, epoch):
    st, flags, timeouts = cp.cp_meta_status(meta)
    assert st == cp.CP_OK and timeouts == 0, (st, hex(flags), timeouts)
    ref = oracle_full(grads, cu, W, "f32")
    for t in range(2):
        for o in range(W):
            got = to_np(out[t][o])
            assert not np.isnan(got).any()
            assert bits_equal(got, ref[t][1][o]), (t, o)
    assert (epochs == epoch).all()


def test_per_rank_streams_with_delayed_writer(cp):
    """W=2 ranks, each the whole protocol on its own stream; writer 1 is delayed and
    the slots start as NaN.  Owner 0 must wait for writer 1's epoch, so the result
    equals the oracle and holds no NaN."""
    W = 2
    say(f"case per-rank full protocol W={W}")
    cu, grads, meta, slots, out, epochs = per_rank_case(cp, W, 42)
    streams = [torch.cuda.Stream() for _ in range(W)]
    for r in range(W):
        with torch.cuda.stream(streams[r]):
            if r == W - 1:
                torch.cuda._sleep(50_000_000)  # device-side spin before this writer starts
            cp.cp_grad_return(grads, slots, out, meta, rank=r, epochs=epochs, epoch=3,
                              wait_timeout_us=5_000_000, stream=streams[r])
    torch.cuda.synchronize()
    check_per_rank_result(cp, meta, cu, grads, out, epochs, W, 3)


@pytest.mark.parametrize("W", [4, 8])
def test_per_rank_split_phases_with_delayed_writer(cp, W):
    """W ranks on W streams, each enqueueing its writer half (scatter, publish) and
    then its owner half (wait, sum).  Writers' halves are all enqueued before any
    owner half, so ranks whose streams share a hardware queue cannot block each
    other; the delayed last writer still forces every other owner to wait."""
    say(f"case per-rank split phases W={W}")
    cu, grads, meta, slots, out, epochs = per_rank_case(cp, W, 40 + W)
    streams = [torch.cuda.Stream() for _ in range(W)]
    for r in range(W):
        with torch.cuda.stream(streams[r]):
            if r == W - 1:
                torch.cuda._sleep(50_000_000)
            cp.cp_grad_return(grads, slots, out, meta, rank=r, epochs=epochs, epoch=9,
                              phases=cp.CP_PHASE_SCATTER | cp.CP_PHASE_PUBLISH, stream=streams[r])
    for r in range(W):
        cp.cp_grad_return(grads, slots, out, meta, rank=r, epochs=epochs, epoch=9,
                          wait_timeout_us=5_000_000, phases=cp.CP_PHASE_WAIT | cp.CP_PHASE_SUM,
                          stream=streams[r])
    torch.cuda.synchronize()
    check_per_rank_result(cp, meta, cu, grads, out, epochs, W, 9)


def test_repeated_calls_reuse_slots_and_epochs(cp):
    """Twelve gradient returns in a row on the same slots and epoch table (epoch
    1, 2, ...), per-rank split phases on 4 streams with the last writer delayed
    every time and new gradients each time: an owner that stopped waiting early
    would sum the previous call's slots, so every call's output must equal the
    oracle for that call's gradients."""
    W = 4
    say(f"case repeated per-rank calls W={W}")
    cu, grads, meta, slots, out, epochs = per_rank_case(cp, W, 77)
    streams = [torch.cuda.Stream() for _ in range(W)]
    gen = torch.Generator(device=DEV).manual_seed(77)
    for epoch in range(1, 13):
        for t in range(2):
            for w in range(W):
                grads[t][w].copy_(torch.randn(grads[t][w].shape, generator=gen, device=DEV))
        torch.cuda.synchronize()
        for r in range(W):
            with torch.cuda.stream(streams[r]):
                if r == W - 1:
                    torch.cuda._sleep(20_000_000)
                cp.cp_grad_return(grads, slots, out, meta, rank=r, epochs=epochs, epoch=epoch,
                                  phases=cp.CP_PHASE_SCATTER | cp.CP_PHASE_PUBLISH, stream=streams[r])
        for r in range(W):
            cp.cp_grad_return(grads, slots, out, meta, rank=r, epochs=epochs, epoch=epoch,
                              wait_timeout_us=5_000_000, phases=cp.CP_PHASE_WAIT | cp.CP_PHASE_SUM,
                              stream=streams[r])
        torch.cuda.synchronize()
        check_per_rank_result(cp, meta, cu, grads, out, epochs, W, epoch)


def test_wait_blocks_until_host_releases_epoch(cp):
    """Rank 0 of W=2 runs alone: writer 1's slot data is already in place but its epoch
    is withheld.  While rank 0's device wait spins, its output still holds the poison
    (read back through a copy on another stream); once the host writes the epoch, the
    wait ends, the sum runs and equals the oracle, and no timeout is reported."""
    say("case host-released epoch")
    W = 2
    cu = np.array([0, 64, 128], dtype=np.int32)
    grads = [[torch.randn((128, 2, 64), device=DEV) for _ in range(W)]]
    meta = make_meta(cp, cu, 128, W)
    slots, out = alloc(grads, W, torch.float32, fill=float("nan"))
    # writer 1's scatter, done beforehand; its epoch is not published
    ref_slots, ref_out = O.grad_return([to_np(g) for g in grads[0]], cu, W, "f32", "f32")
    slots[0][0][1].copy_(torch.from_numpy(ref_slots[0][1]))
    epochs = torch.zeros((W, W), dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    main, side = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(main):
        cp.cp_grad_return(grads, slots, out, meta, rank=0, epochs=epochs, epoch=4,
                          wait_timeout_us=10_000_000, stream=main)
    import time
    time.sleep(0.2)
    with torch.cuda.stream(side):
        probe = out[0][0].to("cpu")  # copy on the side stream while rank 0 waits
        assert torch.isnan(probe).all(), "the owner summed before every epoch was published"
        release = torch.full((1,), 4, dtype=torch.int32).pin_memory()
        epochs[0, 1:2].copy_(release, non_blocking=True)
    torch.cuda.synchronize()
    st, flags, timeouts = cp.cp_meta_status(meta)
    assert st == cp.CP_OK and timeouts == 0, (st, hex(flags), timeouts)
    assert bits_equal(to_np(out[0][0]), ref_out[0])


def test_epoch_timeout_is_reported_not_hung(cp):
    """Per-rank calls on ONE stream: rank 0 waits for rank 1's epoch, which is queued
    behind it.  The device wait gives up after 2 ms, rank 0's sum writes nothing and
    the timeout is reported; rank 1 then completes normally."""
    say("case epoch timeout")
    W = 2
    cu = np.array([0, 64], dtype=np.int32)
    grads = [[torch.randn((64, 1, 8), device=DEV) for _ in range(W)]]
    meta = make_meta(cp, cu, 64, W)
    slots, out = alloc(grads, W, torch.float32, fill=-7.0)
    epochs = torch.zeros((W, W), dtype=torch.int32, device=DEV)
    for r in range(W):
        cp.cp_grad_return(grads, slots, out, meta, rank=r, epochs=epochs, epoch=1,
                          wait_timeout_us=2000)
    st, flags, timeouts = cp.cp_meta_status(meta)
    assert st == cp.CP_ERR_TIMEOUT and timeouts == 0b01, (st, hex(flags), timeouts)
    assert (out[0][0] == -7.0).all()           # fail-closed: owner 0 wrote nothing
    ref = O.grad_return([to_np(g) for g in grads[0]], cu, W, "f32", "f32")[1]
    assert bits_equal(to_np(out[0][1]), ref[1])
    # a later, correctly ordered call clears the timeout mask
    cp.cp_grad_return(grads, slots, out, meta, epochs=epochs, epoch=2)
    st, flags, timeouts = cp.cp_meta_status(meta)
    assert st == cp.CP_OK and timeouts == 0
    assert bits_equal(to_np(out[0][0]), ref[0])


def test_grad_return_rejects_mismatch(cp):
    cu = np.array([0, 64], dtype=np.int32)
    grads = [[torch.randn((64, 1, 8), device=DEV) for _ in range(2)]]
    m128 = make_meta(cp, np.array([0, 128], dtype=np.int32), 128, 2)  # built for another token count
    slots, out = alloc(grads, 2, torch.float32, fill=3.0)
    cp.cp_grad_return(grads, slots, out, m128)
    st, flags, _ = cp.cp_meta_status(m128)
    assert st == cp.CP_ERR_META and flags & cp.CP_CALL_TOKENS_MISMATCH
    assert (out[0][0] == 3.0).all() and (slots[0][0][1] == 3.0).all()
    m4 = make_meta(cp, cu, 64, 4)
    fused = [[torch.full((32, 1, 8), 3.0, device=DEV) for _ in range(2)]]
    cp.cp_grad_return_fused(grads, fused, m4)  # W=2 call on W=4 metadata
    st, flags, _ = cp.cp_meta_status(m4)
    assert st == cp.CP_ERR_META and flags & cp.CP_CALL_CP_SIZE_MISMATCH
    assert (fused[0][0] == 3.0).all()
    with pytest.raises(cp.CpError) as e:  # output aliasing an input
        cp.cp_grad_return_fused(grads, [[grads[0][0][:32], grads[0][1][32:]]], make_meta(cp, cu, 64, 2))
    assert e.value.status == cp.CP_ERR_ALIAS


# ------------------------------------------------------------------ largest sizes
def test_largest_sizes(cp):
    """Fused gradient return at T = 2^31 - 8 tokens (W = 2, rows of 4 fp32) and a
    slot sum over 2^31 + 5 elements: every offset past 2^31 elements is computed in
    64 bits.  Sampled rows / elements against the oracle's map and sum."""
    T, W = (1 << 31) - 8, 2
    say(f"case largest sizes: fused T={T}, slot sum n={(1 << 31) + 5}")
    cu = np.array([0, T], dtype=np.int32)
    gen = torch.Generator(device=DEV).manual_seed(2)
    grads = [[torch.randn((T, 1, 4), generator=gen, device=DEV) for _ in range(W)]]
    meta = make_meta(cp, cu, T, W)
    n = T // W
    out = [[torch.empty((n, 1, 4), device=DEV) for _ in range(W)]]
    cp.cp_grad_return_fused(grads, out, meta)
    rng = np.random.default_rng(9)
    for o in range(W):
        idx = np.unique(np.concatenate([rng.integers(0, n, size=300), [0, n - 1]]))
        g = torch.tensor([O.rank_row(cu, T, W, O.DUAL_CHUNK_SWAP, o, int(i)) for i in idx], device=DEV)
        src = [to_np(grads[0][w].index_select(0, g)) for w in range(W)]
        ref = O.slot_sum(src, "f32", "f32")
        assert bits_equal(to_np(out[0][o].index_select(0, torch.from_numpy(idx).to(DEV))), ref), o
    assert cp.cp_meta_status(meta)[0] == cp.CP_OK
    del grads, out
    torch.cuda.empty_cache()
    m = (1 << 31) + 5
    slots = [torch.randn(m, generator=gen, device=DEV) for _ in range(2)]
    res = torch.empty(m, device=DEV)
    cp.cp_slot_sum(slots, res)
    idx = np.unique(np.concatenate([rng.integers(0, m, size=2000), [0, (1 << 31) - 1, 1 << 31, m - 1]]))
    ti = torch.from_numpy(idx).to(DEV)
    ref = O.slot_sum([to_np(s.index_select(0, ti)) for s in slots], "f32", "f32")
    assert bits_equal(to_np(res.index_select(0, ti)), ref)
    del slots, res
    torch.cuda.empty_cache()
