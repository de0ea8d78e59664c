"""cp_grad_return_noalloc (owner slots in the library's static device workspace)
against cp_grad_return (caller-allocated slots), through the C ABI: bit-for-bit
equal outputs on consecutive calls of falling size, both policies, fp32 and
bf16, overwrite and accumulate; a call beyond the workspace is refused on the
host and writes nothing."""
import ctypes
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from gpu_util import DEV, O, bits_equal, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cp():
    from thd_token_layout_amd import cpthd
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return cpthd


def table(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def noalloc(cp, grads, out, meta, accumulate=False):
    """The C entry point itself, on torch's current stream."""
    n_t, W = len(grads), len(grads[0])
    T, H, D = grads[0][0].shape
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return cp.lib.cp_grad_return_noalloc(W, n_t, table([g for row in grads for g in row]),
                                         table([o for row in out for o in row]), T, H, D,
                                         cp.dtype_code(grads[0][0].dtype), cp.dtype_code(out[0][0].dtype),
                                         meta.ptr(), cp.CP_SUM_ACCUMULATE if accumulate else 0, stream)


def case(cp, W, lengths, H, D, in_dt, out_dt, policy, n_tensors, accumulate, seed):
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    n = T // W
    say(f"case noalloc W={W} T={T} [{H},{D}] {in_dt}->{out_dt} policy={policy} tensors={n_tensors} "
        f"accumulate={accumulate}")
    meta = cp.cp_build_meta(torch.from_numpy(cu).to(DEV), T, W, policy, check=True)
    gen = torch.Generator(device=DEV).manual_seed(seed)
    grads = [[torch.randn((T, H, D), generator=gen, device=DEV).to(in_dt) for _ in range(W)]
             for _ in range(n_tensors)]
    start = [[torch.randn((n, H, D), generator=gen, device=DEV).to(out_dt) for _ in range(W)]
             for _ in range(n_tensors)]
    # the existing entry point, with caller-allocated slots
    ref = [[s.clone() for s in row] for row in start]
    slots = [[[torch.empty((n, H, D), dtype=in_dt, device=DEV) for _ in range(W)] for _ in range(W)]
             for _ in range(n_tensors)]
    cp.cp_grad_return(grads, slots, ref, meta, accumulate=accumulate)
    # the no-allocation variant
    got = [[s.clone() for s in row] for row in start]
    assert noalloc(cp, grads, got, meta, accumulate) == cp.CP_OK
    torch.cuda.synchronize()
    assert cp.cp_meta_status(meta)[0] == cp.CP_OK
    pol = O.DUAL_CHUNK_SWAP if policy == cp.CP_POLICY_DUAL_CHUNK_SWAP else O.PACKED_CONTIGUOUS
    tag = {torch.float32: "f32", torch.bfloat16: "bf16"}
    for t in range(n_tensors):
        oracle = O.grad_return([to_np(g) for g in grads[t]], cu, W, tag[in_dt], tag[out_dt], policy=pol,
                               into=[to_np(s) for s in start[t]] if accumulate else None)[1]
        for o in range(W):
            assert bits_equal(to_np(got[t][o]), to_np(ref[t][o])), (t, o)
            assert bits_equal(to_np(got[t][o]), oracle[o]), (t, o)


def test_noalloc_equals_grad_return_on_consecutive_calls(cp):
    # 1. the largest case: 2 tensors x 16 slots of 2 MiB = exactly the 64 MiB workspace
    case(cp, 4, [1024, 0, 2048, 1024], 4, 128, torch.float32, torch.float32,
         cp.CP_POLICY_DUAL_CHUNK_SWAP, 2, False, 1)
    # 2. smaller, the other policy, accumulating: the workspace still holds call 1's slots
    case(cp, 2, [7, 0, 41, 48], 2, 8, torch.float32, torch.float32, cp.CP_POLICY_PACKED_CONTIGUOUS, 1, True, 2)
    # 3. smaller still, bf16 in and out, W = 8 (short rows: the scalar paths)
    case(cp, 8, [16, 32, 0, 16], 1, 24, torch.bfloat16, torch.bfloat16, cp.CP_POLICY_DUAL_CHUNK_SWAP, 2,
         False, 3)


def test_noalloc_refuses_more_than_the_workspace(cp):
    W, H, D = 4, 1, 64  # 256-byte fp32 rows
    rows = cp.CP_NOALLOC_SCRATCH_BYTES // (W * W * 256) + 1
    T = W * rows
    meta = cp.cp_build_meta(torch.tensor([0, T], dtype=torch.int32, device=DEV), T, W,
                            cp.CP_POLICY_PACKED_CONTIGUOUS, check=True)
    grads = [[torch.ones((T, H, D), device=DEV) for _ in range(W)]]
    out = [[torch.full((rows, H, D), 7.0, device=DEV) for _ in range(W)]]
    assert noalloc(cp, grads, out, meta) == cp.CP_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert all((o == 7.0).all() for o in out[0])  # nothing was launched
    with pytest.raises(cp.CpError) as e:
        cp.cp_grad_return_noalloc(grads, out, meta)
    assert e.value.status == cp.CP_ERR_TOO_LARGE


def test_noalloc_captured_in_a_graph(cp):
    """The use it exists for: captured in a HIP graph (torch.cuda.CUDAGraph), then
    replayed four times with new gradients written eagerly between replays and other
    eager work in between; every replay equals cp_grad_return run eagerly on the same
    inputs, bit for bit.  The call records only kernel launches."""
    W, H, D, T = 4, 4, 128, 256
    cu = np.array([0, 64, 64, 192, 256], dtype=np.int32)
    n = T // W
    say("case noalloc graph capture and replay")
    meta = cp.cp_build_meta(torch.from_numpy(cu).to(DEV), T, W, cp.CP_POLICY_DUAL_CHUNK_SWAP, check=True)
    grads = [[torch.empty((T, H, D), device=DEV) for _ in range(W)] for _ in range(2)]
    got = [[torch.empty((n, H, D), device=DEV) for _ in range(W)] for _ in range(2)]
    ref = [[torch.empty((n, H, D), device=DEV) for _ in range(W)] for _ in range(2)]
    slots = [[[torch.empty((n, H, D), device=DEV) for _ in range(W)] for _ in range(W)] for _ in range(2)]
    gen = torch.Generator(device=DEV).manual_seed(5)

    def fresh():
        for row in grads:
            for g in row:
                g.copy_(torch.randn(g.shape, generator=gen, device=DEV))

    fresh()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        assert noalloc(cp, grads, got, meta) == cp.CP_OK  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        assert noalloc(cp, grads, got, meta) == cp.CP_OK
    for replay in range(4):
        fresh()
        a = torch.randn((256, 256), generator=gen, device=DEV)
        (a @ a).sum().item()  # unrelated eager work and a synchronization between replays
        for row in got:
            for o in row:
                o.fill_(float("nan"))
        graph.replay()
        cp.cp_grad_return(grads, slots, ref, meta)
        torch.cuda.synchronize()
        assert cp.cp_meta_status(meta)[0] == cp.CP_OK
        for t in range(2):
            for o in range(W):
                assert bits_equal(to_np(got[t][o]), to_np(ref[t][o])), (replay, t, o)


def test_noalloc_first_call_under_capture():
    """The one-time lookup of the workspace's device address also works when a process's
    first call is made under graph capture (in a child process, so the call really is its
    first)."""
    say("case noalloc first call under capture (child process)")
    child = os.path.join(os.path.dirname(os.path.abspath(__file__)), "noalloc_capture_child.py")
    res = subprocess.run([sys.executable, child], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-2000:]
    assert "first call captured ok" in res.stdout, res.stdout[-2000:]
