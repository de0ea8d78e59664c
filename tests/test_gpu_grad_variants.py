"""GPU parity of the gradient-return variants against the CPU oracle: the
accumulate mode (the owner's current gradient seeds the fixed-order sum) and
the gradient return under packed-contiguous ownership, through the unfused
protocol, the fused scatter+sum and the plain slot sum.  Bit-exact at
oracle-sized shapes (scalar and vector paths, every dtype pair, ragged rows),
the order and signed-zero pins on the device, the split per-rank protocol, and
sampled rows at the S=262144 fp32 shape."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, O, bits_equal, say, to_np

pytestmark = pytest.mark.gpu

TAG = {torch.float32: "f32", torch.bfloat16: "bf16"}
POL = {"dcs": (0, O.DUAL_CHUNK_SWAP), "pc": (1, O.PACKED_CONTIGUOUS)}


@pytest.fixture(scope="module")
def cp():
    from thd_token_layout_amd import cpthd
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return cpthd


def make_meta(cp, cu_np, T, W, pol):
    cu = torch.from_numpy(np.asarray(cu_np, dtype=np.int32)).to(DEV)
    return cp.cp_build_meta(cu, T, W, POL[pol][0], check=True)


def documents(pol, W, seed, unit=1, count=7, extra=4):
    """Random document lengths valid for the policy: multiples of 2W under
    dual-chunk-swap; any lengths (some empty) under packed-contiguous, with the
    last document padded so that T is a multiple of W (and of `unit`)."""
    rng = np.random.default_rng(seed)
    if pol == "dcs":
        lengths = (rng.integers(0, 6, size=count) * 2 * W * unit).tolist()
        lengths[-1] += 2 * W * unit * extra
    else:
        lengths = rng.integers(0, 40 * unit, size=count).tolist()
        lengths[-1] += W * unit * extra
        lengths[-1] += (-sum(lengths)) % (W * unit)
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def randn(shape, dt, gen, scale=1e-3):
    return (torch.randn(shape, generator=gen, device=DEV) * scale).to(dt)


def run_variants(cp, grads, into, cu, W, pol, accumulate):
    """Unfused (all ranks) and fused results, both starting from `into`."""
    T = grads[0][0].shape[0]
    meta = make_meta(cp, cu, T, W, pol)
    slots = [[[torch.full((T // W,) + tuple(grads[0][0].shape[1:]), float("nan"), device=DEV)
               .to(grads[0][0].dtype) for _ in range(W)] for _ in range(W)] for _ in grads]
    out = [[x.clone() for x in row] for row in into]
    fused = [[x.clone() for x in row] for row in into]
    cp.cp_grad_return(grads, slots, out, meta, accumulate=accumulate)
    cp.cp_grad_return_fused(grads, fused, meta, accumulate=accumulate)
    st = cp.cp_meta_status(meta)
    assert st[0] == cp.CP_OK, st
    return slots, out, fused


def check_against_oracle(grads, into, cu, W, pol, accumulate, slots, out, fused):
    for t in range(len(grads)):
        gn = [to_np(g) for g in grads[t]]
        iv = [to_np(x) for x in into[t]] if accumulate else None
        in_tag, out_tag = TAG[grads[t][0].dtype], TAG[into[t][0].dtype]
        ref_slots, ref_out = O.grad_return(gn, cu, W, in_tag, out_tag, policy=POL[pol][1], into=iv)
        ref_fused = O.grad_return_fused(gn, cu, W, in_tag, out_tag, policy=POL[pol][1], into=iv)
        for o in range(W):
            for w in range(W):
                assert bits_equal(to_np(slots[t][o][w]), ref_slots[o][w]), (t, o, w)
            assert bits_equal(to_np(out[t][o]), ref_out[o]), (t, o)
            assert bits_equal(to_np(fused[t][o]), ref_fused[o]), (t, o)


CASES = [
    # (W, H, D, in dtype, out dtype): [3,40] rows take the scalar paths, [4,128]
    # and wider the vector paths (whole 512-element groups for fp32 data).
    (2, 3, 40, torch.float32, torch.float32), (3, 3, 40, torch.bfloat16, torch.bfloat16),
    (4, 4, 128, torch.float32, torch.float32), (4, 8, 128, torch.float32, torch.bfloat16),
    (4, 4, 128, torch.bfloat16, torch.float32), (8, 4, 128, torch.bfloat16, torch.bfloat16),
    (8, 16, 128, torch.float32, torch.float32), (2, 20, 128, torch.bfloat16, torch.bfloat16),
    (5, 3, 8, torch.float32, torch.float32), (16, 1, 16, torch.bfloat16, torch.bfloat16),
]


@pytest.mark.parametrize("pol", ["dcs", "pc"])
@pytest.mark.parametrize("W,H,D,in_dt,out_dt", CASES)
def test_accumulate(cp, pol, W, H, D, in_dt, out_dt):
    say(f"case accumulate {pol} W={W} [{H},{D}] {in_dt}->{out_dt}")
    cu = documents(pol, W, seed=W * 31 + H, unit=8)
    T = int(cu[-1])
    gen = torch.Generator(device=DEV).manual_seed(W + H + D)
    grads = [[randn((T, H, D), in_dt, gen) for _ in range(W)] for _ in range(2)]
    into = [[randn((T // W, H, D), out_dt, gen) for _ in range(W)] for _ in range(2)]
    slots, out, fused = run_variants(cp, grads, into, cu, W, pol, accumulate=True)
    check_against_oracle(grads, into, cu, W, pol, True, slots, out, fused)


@pytest.mark.parametrize("W,H,D,in_dt,out_dt", CASES)
def test_packed_contiguous_grad_return(cp, W, H, D, in_dt, out_dt):
    say(f"case pc grad return W={W} [{H},{D}] {in_dt}->{out_dt}")
    cu = documents("pc", W, seed=W * 7 + D, extra=30)
    T = int(cu[-1])
    gen = torch.Generator(device=DEV).manual_seed(3 * W + D)
    grads = [[randn((T, H, D), in_dt, gen) for _ in range(W)] for _ in range(2)]
    into = [[torch.full((T // W, H, D), 5.0, dtype=out_dt, device=DEV) for _ in range(W)] for _ in range(2)]
    slots, out, fused = run_variants(cp, grads, into, cu, W, "pc", accumulate=False)
    check_against_oracle(grads, into, cu, W, "pc", False, slots, out, fused)


@pytest.mark.parametrize("n,W,in_dt,out_dt,offset", [
    (1, 8, torch.float32, torch.float32, 0), (7, 3, torch.float32, torch.bfloat16, 0),
    (1000003, 8, torch.float32, torch.float32, 0), (4099, 5, torch.bfloat16, torch.bfloat16, 0),
    (4099, 5, torch.bfloat16, torch.float32, 0), (777, 4, torch.float32, torch.float32, 1),
    (777, 4, torch.bfloat16, torch.bfloat16, 3), (65536, 64, torch.float32, torch.float32, 0)])
def test_slot_sum_accumulate(cp, n, W, in_dt, out_dt, offset):
    say(f"case slot sum accumulate n={n} W={W} {in_dt}->{out_dt} offset={offset}")
    gen = torch.Generator(device=DEV).manual_seed(n + 2 * W)
    slots = [torch.randn(n + offset, generator=gen, device=DEV).to(in_dt)[offset:] for _ in range(W)]
    base = torch.randn(n + offset, generator=gen, device=DEV).to(out_dt)[offset:]
    into = to_np(base)
    cp.cp_slot_sum(slots, base, accumulate=True)
    ref = O.slot_sum([to_np(s) for s in slots], TAG[in_dt], TAG[out_dt], into=into)
    assert bits_equal(to_np(base), ref)


def test_accumulate_order_and_signed_zero(cp):
    """1e8 accumulated with slots (1, -1e8, 1) gives 1 only in the sequential order;
    -0 into -0 slots stays -0, +0 into -0 slots gives +0."""
    say("case accumulate order pin")
    vals = [1.0, -1e8, 1.0]
    for pol in ("dcs", "pc"):
        cu = np.array([0, 48], dtype=np.int32)
        grads = [[torch.full((48, 1, 8), v, device=DEV) for v in vals]]
        into = [[torch.full((16, 1, 8), 1e8, device=DEV) for _ in range(3)]]
        _, out, fused = run_variants(cp, grads, into, cu, 3, pol, accumulate=True)
        for o in range(3):
            assert (out[0][o] == 1.0).all() and (fused[0][o] == 1.0).all(), (pol, o)
        nz = [[torch.full((48, 1, 8), -0.0, device=DEV) for _ in range(3)]]
        for seed, want in ((-0.0, -2**31), (0.0, 0)):
            into = [[torch.full((16, 1, 8), seed, device=DEV) for _ in range(3)]]
            _, out, fused = run_variants(cp, nz, into, cu, 3, pol, accumulate=True)
            for o in range(3):
                assert (out[0][o].view(torch.int32) == want).all() and \
                    (fused[0][o].view(torch.int32) == want).all(), (pol, seed, o)
    ss = torch.full((1000,), 1e8, device=DEV)
    cp.cp_slot_sum([torch.full((1000,), v, device=DEV) for v in vals], ss, accumulate=True)
    assert (ss == 1.0).all()


@pytest.mark.parametrize("pol,W", [("dcs", 4), ("pc", 4), ("pc", 3)])
def test_accumulate_per_rank_split_phases(cp, pol, W):
    """Per-rank protocol on one stream: every writer's SCATTER|PUBLISH half, then
    every owner's WAIT|SUM half with the accumulate flag; slots start as NaN."""
    say(f"case per-rank split phases accumulate {pol} W={W}")
    cu = documents(pol, W, seed=90 + W, unit=16)
    T = int(cu[-1])
    gen = torch.Generator(device=DEV).manual_seed(90 + W)
    grads = [[randn((T, 4, 64), torch.float32, gen) for _ in range(W)] for _ in range(2)]
    into = [[randn((T // W, 4, 64), torch.float32, gen) for _ in range(W)] for _ in range(2)]
    meta = make_meta(cp, cu, T, W, pol)
    slots = [[[torch.full((T // W, 4, 64), float("nan"), device=DEV) for _ in range(W)] for _ in range(W)]
             for _ in range(2)]
    out = [[x.clone() for x in row] for row in into]
    epochs = torch.zeros((W, W), dtype=torch.int32, device=DEV)
    for r in range(W):
        cp.cp_grad_return(grads, slots, out, meta, rank=r, epochs=epochs, epoch=3,
                          phases=cp.CP_PHASE_SCATTER | cp.CP_PHASE_PUBLISH, accumulate=True)
    for r in range(W):
        cp.cp_grad_return(grads, slots, out, meta, rank=r, epochs=epochs, epoch=3,
                          phases=cp.CP_PHASE_WAIT | cp.CP_PHASE_SUM, accumulate=True)
    st, flags, timeouts = cp.cp_meta_status(meta)
    assert st == cp.CP_OK and timeouts == 0, (st, hex(flags), timeouts)
    for t in range(2):
        ref = O.grad_return([to_np(g) for g in grads[t]], cu, W, "f32", "f32", policy=POL[pol][1],
                            into=[to_np(x) for x in into[t]])[1]
        for o in range(W):
            assert bits_equal(to_np(out[t][o]), ref[o]), (t, o)


def test_s256k_w4_packed_contiguous_and_accumulate(cp):
    """S=262144, W=4, 4 x {dK, dV} [S,20,128] fp32 under packed-contiguous metadata
    with the documents of the layout workload: unfused with epochs, sampled rows
    against the oracle; fused == unfused; fused accumulate, sampled rows."""
    from thd_token_layout_amd import workloads as WL
    say("case s256k W=4 packed-contiguous grad return + accumulate (full size)")
    w = WL.WORKLOADS["pc_s256k_w4"]
    cu = WL.cu_seqlens(w)
    W, T, H, D = 4, w.total_tokens, 20, 128
    n = T // W
    gen = torch.Generator(device=DEV).manual_seed(256)
    grads = [[randn((T, H, D), torch.float32, gen) for _ in range(W)] for _ in range(2)]
    meta = make_meta(cp, cu, T, W, "pc")
    slots = [[[torch.empty((n, H, D), device=DEV) for _ in range(W)] for _ in range(W)] for _ in range(2)]
    out = [[torch.empty((n, H, D), device=DEV) for _ in range(W)] for _ in range(2)]
    epochs = torch.zeros((W, W), dtype=torch.int32, device=DEV)
    cp.cp_grad_return(grads, slots, out, meta, epochs=epochs, epoch=1)
    assert cp.cp_meta_status(meta)[0] == cp.CP_OK
    rng = np.random.default_rng(1)
    idx = np.unique(np.concatenate([rng.integers(0, n, size=256), [0, n - 1]]))
    lidx = torch.from_numpy(idx).to(DEV)
    for t in range(2):
        for o in range(W):
            gidx = torch.from_numpy(O.rank_rows(cu, T, W, O.PACKED_CONTIGUOUS, o)[idx]).to(DEV)
            src = [to_np(grads[t][w_].index_select(0, gidx)) for w_ in range(W)]
            assert bits_equal(to_np(out[t][o].index_select(0, lidx)), O.slot_sum(src, "f32", "f32"))
            for w_ in range(W):
                assert bits_equal(to_np(slots[t][o][w_].index_select(0, lidx)), src[w_])
    del slots
    torch.cuda.empty_cache()
    fused = [[torch.empty_like(x) for x in row] for row in out]
    cp.cp_grad_return_fused(grads, fused, meta)
    torch.cuda.synchronize()
    for t in range(2):
        for o in range(W):
            assert torch.equal(fused[t][o].view(torch.int32), out[t][o].view(torch.int32)), (t, o)
    # accumulate into the unfused result
    cp.cp_grad_return_fused(grads, out, meta, accumulate=True)
    for t in range(2):
        for o in range(W):
            gidx = torch.from_numpy(O.rank_rows(cu, T, W, O.PACKED_CONTIGUOUS, o)[idx]).to(DEV)
            src = [to_np(grads[t][w_].index_select(0, gidx)) for w_ in range(W)]
            ref = O.slot_sum(src, "f32", "f32", into=to_np(fused[t][o].index_select(0, lidx)))
            assert bits_equal(to_np(out[t][o].index_select(0, lidx)), ref), (t, o)
    del grads, out, fused
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n_tensors", [1, 3, 5])
def test_any_number_of_gradient_tensors(cp, n_tensors):
    """The gradient return takes any number of tensors per rank (dK, dV, ... ): one
    table row per tensor, every one bit-exact against the oracle."""
    say(f"case {n_tensors} gradient tensors per rank")
    W, H, D = 4, 2, 128
    cu = documents("dcs", W, seed=n_tensors, unit=8)
    T = int(cu[-1])
    gen = torch.Generator(device=DEV).manual_seed(500 + n_tensors)
    grads = [[randn((T, H, D), torch.float32, gen) for _ in range(W)] for _ in range(n_tensors)]
    into = [[randn((T // W, H, D), torch.bfloat16, gen) for _ in range(W)] for _ in range(n_tensors)]
    slots, out, fused = run_variants(cp, grads, into, cu, W, "dcs", accumulate=False)
    check_against_oracle(grads, into, cu, W, "dcs", False, slots, out, fused)
