"""GPU parity of the all-reduce of W rank buffers (one-shot, ring, two-shot and the
ring in one launch), through the C ABI, bit-exact against the CPU oracle: every
rank's output, for every rank count, size (empty and short chunks, ragged tails,
unaligned views), dtype and the W = 8, 1 KiB - 16 MiB sizes of the latency sweep;
special values; errors the host rejects; the launch-per-step algorithms captured
in a HIP graph and replayed."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import DEV, O, bits_equal, say, to_np

pytestmark = pytest.mark.gpu

TAG = {torch.float32: "f32", torch.bfloat16: "bf16"}
REF = {"one_shot": O.allreduce_one_shot, "ring": O.allreduce_ring, "two_shot": O.allreduce_two_shot}


@pytest.fixture(scope="module")
def cp():
    from thd_token_layout_amd import cpthd
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return cpthd


def rank_inputs(W, n, dtype, seed, offset=0):
    """W input views of n elements (offset elements into their allocation)."""
    gen = torch.Generator(device=DEV).manual_seed(seed)
    full = [torch.randn(n + offset, generator=gen, device=DEV).to(dtype) for _ in range(W)]
    return [f[offset:] for f in full]


def nan_outputs(W, n, dtype, offset=0):
    return [torch.full((n + offset,), float("nan"), dtype=dtype, device=DEV)[offset:] for _ in range(W)]


def check(cp, algo, xs, outs):
    ref = REF[algo]([to_np(x) for x in xs], TAG[xs[0].dtype])
    for r, o in enumerate(outs):
        assert bits_equal(to_np(o), ref[r]), (algo, r)


@pytest.mark.parametrize("algo", ["one_shot", "ring", "two_shot"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("W,n", [(1, 1000), (2, 1), (2, 130), (3, 64), (3, 65), (4, 511), (4, 512),
                                 (5, 4099), (8, 256), (8, 300), (8, 4096), (8, 100003), (16, 1 << 16),
                                 (7, 3 * 512 * 7 + 5), (64, 70000)])
def test_allreduce_matches_oracle(cp, algo, dtype, W, n):
    say(f"case allreduce {algo} W={W} n={n} {dtype}")
    xs = rank_inputs(W, n, dtype, seed=W * 1000 + n)
    outs = nan_outputs(W, n, dtype)
    cp.cp_allreduce(xs, outs, algo=algo)
    torch.cuda.synchronize()
    check(cp, algo, xs, outs)


@pytest.mark.parametrize("algo", ["one_shot", "ring", "two_shot"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("offset", [1, 2, 3])
def test_unaligned_views(cp, algo, dtype, offset):
    """Views that start off a 16-byte boundary take the element path."""
    W, n = 4, 2000 + offset
    say(f"case allreduce unaligned {algo} {dtype} offset={offset}")
    xs = rank_inputs(W, n, dtype, seed=offset, offset=offset)
    outs = nan_outputs(W, n, dtype, offset=(offset + 1) % 4)
    cp.cp_allreduce(xs, outs, algo=algo)
    torch.cuda.synchronize()
    check(cp, algo, xs, outs)


@pytest.mark.parametrize("algo", ["one_shot", "ring", "two_shot"])
@pytest.mark.parametrize("size", [1024 << k for k in range(15)])
def test_sweep_sizes(cp, algo, size):
    """W = 8 fp32 buffers of 1 KiB ... 16 MiB, as timed by the benchmark."""
    W, n = 8, size // 4
    say(f"case allreduce sweep {algo} bytes={size}")
    xs = rank_inputs(W, n, torch.float32, seed=size)
    outs = nan_outputs(W, n, torch.float32)
    cp.cp_allreduce(xs, outs, algo=algo)
    torch.cuda.synchronize()
    check(cp, algo, xs, outs)


@pytest.mark.parametrize("seed", range(48))
def test_random_configurations(cp, seed):
    """Seeded random rank counts, sizes, dtypes, algorithms (one-shot, ring, ring in one
    launch) and view offsets."""
    rng = np.random.default_rng(5000 + seed)
    W = int(rng.choice([1, 2, 3, 4, 6, 8, 11, 16, 32]))
    n = int(rng.choice([int(rng.integers(0, 200)), int(rng.integers(200, 5000)), int(rng.integers(5000, 300000))]))
    dtype = [torch.float32, torch.bfloat16][int(rng.integers(0, 2))]
    algo = ["one_shot", "ring", "two_shot", "ring_one_launch"][int(rng.integers(0, 4))]
    off_in, off_out = (int(v) for v in rng.choice([0, 0, 0, 1, 3], size=2))
    say(f"case allreduce random seed={seed}: {algo} W={W} n={n} {dtype} offsets={off_in},{off_out}")
    xs = rank_inputs(W, n, dtype, seed=seed, offset=off_in)
    outs = nan_outputs(W, n, dtype, offset=off_out)
    if algo == "ring_one_launch":
        sig = torch.zeros(cp.cp_allreduce_signal_bytes(W), dtype=torch.uint8, device=DEV)
        cp.cp_allreduce_signal(xs, sig, epoch=seed + 1, outs=outs, wait_timeout_us=500000)
        assert cp.cp_allreduce_signal_status(sig, W, seed + 1) == cp.CP_OK
        algo = "ring"  # same result as the launch-per-step ring
    else:
        cp.cp_allreduce(xs, outs, algo=algo)
    torch.cuda.synchronize()
    check(cp, algo, xs, outs)


@pytest.mark.parametrize("algo", ["one_shot", "ring", "two_shot", "ring_one_launch"])
def test_special_values(cp, algo):
    """Signed zeros, infinities, NaN, overflow to inf, denormals; NaN results are
    compared as NaN (payloads of two NaNs meeting are not fixed by IEEE)."""
    W, n = 4, 1024
    say(f"case allreduce special values {algo}")
    vals = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 3.0e38, -3.0e38, 1e-45, -1e-45, 1.0], dtype=np.float32)
    rng = np.random.default_rng(9)
    host = [vals[rng.integers(0, len(vals), size=n)] for _ in range(W)]
    host[0][:64] = -0.0
    host[1][:64] = -0.0
    host[2][:64] = -0.0
    host[3][:64] = -0.0
    xs = [torch.from_numpy(h).to(DEV) for h in host]
    outs = nan_outputs(W, n, torch.float32)
    if algo == "ring_one_launch":
        sig = torch.zeros(cp.cp_allreduce_signal_bytes(W), dtype=torch.uint8, device=DEV)
        cp.cp_allreduce_signal(xs, sig, epoch=1, outs=outs, wait_timeout_us=500000)
        assert cp.cp_allreduce_signal_status(sig, W, 1) == cp.CP_OK
        algo = "ring"
    else:
        cp.cp_allreduce(xs, outs, algo=algo)
    torch.cuda.synchronize()
    ref = REF[algo](host, "f32")
    for r in range(W):
        got = to_np(outs[r])
        nan = np.isnan(ref[r])
        assert (np.isnan(got) == nan).all()
        assert bits_equal(got[~nan], ref[r][~nan]), r
        assert (got[:64].view(np.uint32) == 0x80000000).all()  # -0 + -0 + ... stays -0


def test_shared_input_buffer(cp):
    """Inputs may share memory (they are only read)."""
    say("case allreduce shared input")
    x = rank_inputs(1, 5000, torch.float32, seed=3)[0]
    xs = [x, x, x]
    for algo in ("one_shot", "ring", "two_shot"):
        outs = nan_outputs(3, 5000, torch.float32)
        cp.cp_allreduce(xs, outs, algo=algo)
        torch.cuda.synchronize()
        check(cp, algo, xs, outs)


def test_repeated_calls_overwrite(cp):
    """A second call with new inputs and fewer elements gives that call's result."""
    say("case allreduce repeated calls")
    W = 8
    outs = nan_outputs(W, 10000, torch.float32)
    for algo in ("one_shot", "ring", "two_shot"):
        for n, seed in ((10000, 1), (6001, 2)):
            xs = rank_inputs(W, n, torch.float32, seed=seed)
            view = [o[:n] for o in outs]
            cp.cp_allreduce(xs, view, algo=algo)
            torch.cuda.synchronize()
            check(cp, algo, xs, view)


def test_errors_rejected_before_launch(cp):
    say("case allreduce errors")
    lib = cp.lib
    W, n = 4, 1000
    xs = rank_inputs(W, n, torch.float32, seed=5)
    outs = nan_outputs(W, n, torch.float32)
    tab = lambda ts: (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])  # noqa: E731
    for algo in (cp.CP_ALLREDUCE_ONE_SHOT, cp.CP_ALLREDUCE_RING, cp.CP_ALLREDUCE_TWO_SHOT):
        # an output that is an input, or two outputs that overlap
        assert lib.cp_allreduce(algo, W, tab(xs), tab([xs[1]] + outs[1:]), n, cp.CP_F32, None) == cp.CP_ERR_ALIAS
        assert lib.cp_allreduce(algo, W, tab(xs), tab([outs[0], outs[0][10:]] + outs[2:]), n - 10,
                                cp.CP_F32, None) == cp.CP_ERR_ALIAS
        # sizes that run past the end of the buffers' allocations (2^36 elements:
        # more than any allocation on the device)
        assert lib.cp_allreduce(algo, W, tab(xs), tab(outs), 1 << 36, cp.CP_F32, None) == cp.CP_ERR_SHAPE
        # host memory
        host = torch.empty(n)
        assert lib.cp_allreduce(algo, W, tab(xs), tab(outs[:3] + [host]), n, cp.CP_F32, None) == cp.CP_ERR_DEVICE
    torch.cuda.synchronize()
    assert all(torch.isnan(o).all() for o in outs), "a rejected call wrote an output"
    with pytest.raises(ValueError):
        cp.cp_allreduce(xs, outs[:3])


@pytest.mark.parametrize("algo", ["one_shot", "ring", "two_shot"])
def test_graph_capture_replays(cp, algo):
    """Both algorithms record only kernel launches: captured once, replayed with
    new inputs written eagerly between replays, every replay is exact."""
    W, n = 8, 70000
    say(f"case allreduce graph {algo}")
    xs = [torch.empty(n, device=DEV) for _ in range(W)]
    outs = [torch.empty(n, device=DEV) for _ in range(W)]
    gen = torch.Generator(device=DEV).manual_seed(17)

    def fresh():
        for x in xs:
            x.copy_(torch.randn(n, generator=gen, device=DEV))

    fresh()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        cp.cp_allreduce(xs, outs, algo=algo)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cp.cp_allreduce(xs, outs, algo=algo)
    for replay in range(3):
        fresh()
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        check(cp, algo, xs, outs)


# ------------------------------------------------------------------ the ring in one launch
def signal_buffer(cp, W):
    return torch.zeros(cp.cp_allreduce_signal_bytes(W), dtype=torch.uint8, device=DEV)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("W,n", [(1, 1000), (2, 1), (2, 130), (3, 65), (4, 512), (5, 4099), (8, 256),
                                 (8, 100003), (8, 1 << 22), (16, 1 << 16), (64, 70000)])
def test_signal_ring_matches_oracle(cp, dtype, W, n):
    """Same bits as the launch-per-step ring (the oracle's ring)."""
    say(f"case allreduce one-launch ring W={W} n={n} {dtype}")
    xs = rank_inputs(W, n, dtype, seed=W * 7 + n)
    outs = nan_outputs(W, n, dtype)
    sig = signal_buffer(cp, W)
    cp.cp_allreduce_signal(xs, sig, epoch=1, outs=outs, wait_timeout_us=500000)
    assert cp.cp_allreduce_signal_status(sig, W, 1) == cp.CP_OK
    check(cp, "ring", xs, outs)


@pytest.mark.parametrize("offset", [1, 3])
def test_signal_ring_unaligned(cp, offset):
    W, n = 4, 5000 + offset
    say(f"case allreduce one-launch ring unaligned offset={offset}")
    xs = rank_inputs(W, n, torch.float32, seed=offset, offset=offset)
    outs = nan_outputs(W, n, torch.float32)
    sig = signal_buffer(cp, W)
    cp.cp_allreduce_signal(xs, sig, epoch=3, outs=outs, wait_timeout_us=500000)
    assert cp.cp_allreduce_signal_status(sig, W, 3) == cp.CP_OK
    check(cp, "ring", xs, outs)


def test_signal_ring_repeated_calls_and_stale_epoch(cp):
    """One signal buffer, calls with rising epochs and new inputs: each exact.  A
    call that repeats an epoch finds its flags stale, stops, and is reported."""
    W, n = 8, 300000
    say("case allreduce one-launch ring repeated calls")
    sig = signal_buffer(cp, W)
    outs = nan_outputs(W, n, torch.float32)
    for epoch in (1, 2, 7, 8, 1000):
        xs = rank_inputs(W, n, torch.float32, seed=epoch)
        cp.cp_allreduce_signal(xs, sig, epoch=epoch, outs=outs, wait_timeout_us=500000)
        assert cp.cp_allreduce_signal_status(sig, W, epoch) == cp.CP_OK, epoch
        check(cp, "ring", xs, outs)
    for o in outs:
        o.fill_(float("nan"))
    cp.cp_allreduce_signal(xs, sig, epoch=1000, outs=outs, wait_timeout_us=500000)
    assert cp.cp_allreduce_signal_status(sig, W, 1000) == cp.CP_ERR_ARG
    assert all(torch.isnan(o).all() for o in outs), "a stale call wrote an output"
    cp.cp_allreduce_signal(xs, sig, epoch=1001, outs=outs, wait_timeout_us=500000)
    assert cp.cp_allreduce_signal_status(sig, W, 1001) == cp.CP_OK
    check(cp, "ring", xs, outs)


def test_signal_ring_short_wait_limit_ends(cp):
    """A 1 us wait limit on 16 MiB per rank: the call ends (no hang) and reports
    either success with exact results or a timeout."""
    W, n = 8, 1 << 22
    say("case allreduce one-launch ring 1 us wait limit")
    xs = rank_inputs(W, n, torch.float32, seed=11)
    outs = nan_outputs(W, n, torch.float32)
    sig = signal_buffer(cp, W)
    cp.cp_allreduce_signal(xs, sig, epoch=5, outs=outs, wait_timeout_us=1)
    st = cp.cp_allreduce_signal_status(sig, W, 5)
    say(f"status with a 1 us wait limit: {cp.cp_status_string(st)}")
    assert st in (cp.CP_OK, cp.CP_ERR_TIMEOUT)
    if st == cp.CP_OK:
        check(cp, "ring", xs, outs)
    cp.cp_allreduce_signal(xs, sig, epoch=6, outs=outs, wait_timeout_us=500000)
    assert cp.cp_allreduce_signal_status(sig, W, 6) == cp.CP_OK
    check(cp, "ring", xs, outs)


def test_signal_ring_errors(cp):
    say("case allreduce one-launch ring errors")
    lib = cp.lib
    W, n = 4, 1000
    xs = rank_inputs(W, n, torch.float32, seed=5)
    outs = nan_outputs(W, n, torch.float32)
    sig = signal_buffer(cp, W)
    nb = sig.numel()
    tab = lambda ts: (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])  # noqa: E731
    call = lambda i, o, s, sb, e, dt=cp.CP_F32: lib.cp_allreduce_signal(W, tab(i), tab(o), n, dt, s, sb, e, 0, None)  # noqa: E731
    assert call(xs, outs, sig.data_ptr(), nb, 0) == cp.CP_ERR_ARG                    # epoch 0
    assert call(xs, outs, sig.data_ptr(), nb, 1 << 55) == cp.CP_ERR_ARG              # epoch too large
    assert call(xs, outs, sig.data_ptr(), nb - 1, 1) == cp.CP_ERR_SHAPE              # buffer too small
    assert call(xs, outs, None, nb, 1) == cp.CP_ERR_ARG
    assert call(xs, outs, sig.data_ptr(), nb, 1, cp.CP_F16) == cp.CP_ERR_UNSUPPORTED
    assert call(xs, outs, outs[2].data_ptr(), nb, 1) in (cp.CP_ERR_ALIAS, cp.CP_ERR_SHAPE)  # signals on an output
    assert call(xs, [xs[0]] + outs[1:], sig.data_ptr(), nb, 1) == cp.CP_ERR_ALIAS
    torch.cuda.synchronize()
    assert all(torch.isnan(o).all() for o in outs), "a rejected call wrote an output"
    assert (sig == 0).all()
    assert cp.cp_allreduce_signal_bytes(0) == 0 and cp.cp_allreduce_signal_bytes(65) == 0
    assert lib.cp_allreduce_signal(W, None, None, 0, cp.CP_F32, None, 0, 1, 0, None) == cp.CP_OK  # empty


@pytest.mark.parametrize("algo", ["one_shot", "ring", "two_shot", "ring_one_launch"])
def test_largest_sizes(cp, algo):
    """W = 2 fp32 buffers of 2^31 + 160 elements (8 GiB each): every offset past
    2^31 elements.  With two ranks every algorithm computes x0 + x1 (one fp32 add,
    commutative), checked on sampled elements, chunk edges and the last element."""
    W, n = 2, (1 << 31) + 160
    say(f"case allreduce largest size {algo} n={n}")
    torch.cuda.empty_cache()
    xs = [torch.empty(n, device=DEV) for _ in range(W)]
    gen = torch.Generator(device=DEV).manual_seed(31)
    for x in xs:
        x.normal_(generator=gen)
    outs = [torch.empty(n, device=DEV) for _ in range(W)]
    if algo == "ring_one_launch":
        sig = torch.zeros(cp.cp_allreduce_signal_bytes(W), dtype=torch.uint8, device=DEV)
        cp.cp_allreduce_signal(xs, sig, epoch=1, outs=outs, wait_timeout_us=2000000)
        assert cp.cp_allreduce_signal_status(sig, W, 1) == cp.CP_OK
    else:
        cp.cp_allreduce(xs, outs, algo=algo)
    torch.cuda.synchronize()
    q = O.ring_chunks(n, W)[1][0]
    rng = np.random.default_rng(7)
    idx = np.unique(np.concatenate([rng.integers(0, n, size=2000), [0, q - 1, q, q + 1, n - 2, n - 1],
                                    (1 << 31) + np.arange(-3, 4)]))
    idx_t = torch.from_numpy(idx).to(DEV)
    a, b = (x[idx_t].cpu().numpy() for x in xs)
    want = (a + b).astype(np.float32)
    for r in range(W):
        got = outs[r][idx_t].cpu().numpy()
        assert bits_equal(got, want), r
    del xs, outs
    torch.cuda.empty_cache()


def test_every_small_size(cp):
    """Every n in 0..200 for W = 1..8 (chunk edges, empty chunks, tails of every
    length) under one-shot, ring, two-shot and the ring in one launch, fp32,
    against the oracle; one buffer set reused, outputs poisoned before each call."""
    say("case allreduce every small size")
    gen = torch.Generator(device=DEV).manual_seed(123)
    big_in = [torch.randn(256, generator=gen, device=DEV) for _ in range(8)]
    big_out = [torch.empty(256, device=DEV) for _ in range(8)]
    host_in = [to_np(x) for x in big_in]
    epoch = 0
    for W in range(1, 9):
        say(f"  W={W}")
        sig_w = torch.zeros(cp.cp_allreduce_signal_bytes(W), dtype=torch.uint8, device=DEV)
        first_epoch = epoch + 1
        for n in range(0, 201):
            xs = [x[:n] for x in big_in[:W]]
            outs = [o[:n] for o in big_out[:W]]
            hx = [h[:n] for h in host_in[:W]]
            for algo in ("one_shot", "ring", "two_shot", "ring_one_launch"):
                for o in big_out:
                    o.fill_(float("nan"))
                if algo == "ring_one_launch":
                    epoch += 1
                    cp.cp_allreduce_signal(xs, sig_w, epoch, outs=outs, wait_timeout_us=500000)
                    ref = O.allreduce_ring(hx, "f32")
                else:
                    cp.cp_allreduce(xs, outs, algo=algo)
                    ref = REF[algo](hx, "f32")
                torch.cuda.synchronize()
                for r in range(W):
                    assert bits_equal(to_np(outs[r]), ref[r]), (W, n, algo, r)
        # no call of this W timed out or found a stale epoch
        assert cp.cp_allreduce_signal_status(sig_w, W, first_epoch) == cp.CP_OK
