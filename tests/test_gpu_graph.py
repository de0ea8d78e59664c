"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed:
every replay, with new input values written eagerly between replays and other
eager work in between, equals the oracle.  The library records only kernel
launches (no memset nodes), so a captured sequence replays exactly."""
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


@pytest.mark.parametrize("pol", [0, 1])
def test_captured_sequence_replays(cp, pol):
    say(f"case graph capture and replay, policy={pol}")
    W, H, D = 4, 4, 128
    cu_np = np.array([0, 64, 64, 192, 256], dtype=np.int32) if pol == 0 else \
        np.array([0, 37, 37, 190, 256], dtype=np.int32)
    T = int(cu_np[-1])
    n = T // W
    cu = torch.from_numpy(cu_np).to(DEV)
    meta = cp.cp_build_meta(cu, T, W, pol, check=True)
    attn = cp.cp_build_attn_meta(meta)
    xs = [torch.empty((T, H, D), dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    parts = [torch.empty((W, n, H, D), dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    backs = [torch.empty_like(x) for x in xs]
    grads = [[torch.empty((T, H, D), device=DEV) for _ in range(W)] for _ in range(2)]
    slots = [[[torch.empty((n, H, D), device=DEV) for _ in range(W)] for _ in range(W)] for _ in range(2)]
    out = [[torch.empty((n, H, D), device=DEV) for _ in range(W)] for _ in range(2)]
    fused = [[torch.empty((n, H, D), dtype=torch.bfloat16, device=DEV) for _ in range(W)] for _ in range(2)]
    small = [torch.empty(3000, device=DEV) for _ in range(8)]
    small_out = torch.empty(3000, device=DEV)

    def sequence():
        cp.cp_build_meta(cu, T, W, pol, meta=meta.buf)
        cp.cp_build_attn_meta(meta, attn=attn)
        cp.cp_partition_thd_multi(xs, meta, parts=parts)
        cp.cp_gather_thd_multi(parts, meta, xs=backs)
        cp.cp_grad_return(grads, slots, out, meta)
        cp.cp_grad_return_fused(grads, fused, meta)
        cp.cp_slot_sum(small, small_out)

    gen = torch.Generator(device=DEV).manual_seed(pol)

    def fresh_inputs():
        for x in xs:
            x.copy_(torch.randn(x.shape, generator=gen, device=DEV).to(torch.bfloat16))
        for row in grads:
            for g in row:
                g.copy_(torch.randn(g.shape, generator=gen, device=DEV) * 1e-3)
        for s in small:
            s.copy_(torch.randn(s.shape, generator=gen, device=DEV))

    fresh_inputs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sequence()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sequence()
    ref_attn = O.attention_meta(cu_np, T, W, O.POLICIES[pol])
    for replay in range(4):
        fresh_inputs()
        a = torch.randn((256, 256), generator=gen, device=DEV)
        (a @ a).sum().item()  # unrelated eager work and a synchronization between replays
        for o in out[0]:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert cp.cp_meta_status(meta)[0] == cp.CP_OK
        magic, tables = cp.read_attn_meta(attn, len(cu_np) - 1, W)
        assert magic == cp.CP_ATTN_MAGIC
        for k, v in ref_attn.items():
            assert np.array_equal(tables[k].numpy(), v), (replay, k)
        for x, p, bk in zip(xs, parts, backs):
            assert bits_equal(to_np(p), O.partition(to_np(x), cu_np, W, O.POLICIES[pol])), replay
            assert bits_equal(to_np(bk), to_np(x)), replay
        for t in range(2):
            gn = [to_np(g) for g in grads[t]]
            ref_slots, ref_out = O.grad_return(gn, cu_np, W, "f32", "f32", policy=O.POLICIES[pol])
            ref_fused = O.grad_return_fused(gn, cu_np, W, "f32", "bf16", policy=O.POLICIES[pol])
            for o in range(W):
                assert bits_equal(to_np(out[t][o]), ref_out[o]), (replay, t, o)
                assert bits_equal(to_np(fused[t][o]), ref_fused[o]), (replay, t, o)
        assert bits_equal(to_np(small_out), O.slot_sum([to_np(s) for s in small], "f32", "f32")), replay
