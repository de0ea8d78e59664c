"""GPU parity of the sums' piece layout: 16-byte input pieces with one load in
flight per lane, which serves owner sums and fused gradient returns of at most
four slots (writers) of at least 32 MiB each.  Every dtype pair that has the
layout, ragged tails, the accumulate mode, and both policies with several
documents (row lookups per tile), against the CPU oracle element by element;
eight slots, bf16 -> fp32 and sizes just under the threshold take the batched
units and are compared the same way."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, O, bits_equal, say, to_np

pytestmark = pytest.mark.gpu

TAG = {torch.float32: "f32", torch.bfloat16: "bf16"}
F32, BF16 = torch.float32, torch.bfloat16
PIECE_MIN = 32 << 20  # bytes per slot from which the sums use pieces


@pytest.fixture(scope="module")
def cp():
    from thd_token_layout_amd import cpthd
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return cpthd


def esize(dt):
    return 4 if dt == F32 else 2


SLOT_CASES = [(i, o, W, acc) for i, o in ((F32, F32), (F32, BF16), (BF16, BF16), (BF16, F32))
              for W in (1, 4) for acc in (False, True)] + \
             [(F32, F32, 3, False), (F32, F32, 3, True), (F32, F32, 8, False), (BF16, BF16, 8, True)]


@pytest.mark.parametrize("in_dt,out_dt,W,acc", SLOT_CASES)
def test_slot_sum_pieces(cp, in_dt, out_dt, W, acc):
    """Slots of 32 MiB plus 5 elements (a ragged tail past the whole pieces)."""
    n = PIECE_MIN // esize(in_dt) + 5
    say(f"case slot sum pieces n={n} W={W} {in_dt}->{out_dt} accumulate={acc}")
    gen = torch.Generator(device=DEV).manual_seed(W * 10 + acc)
    slots = [torch.randn(n, generator=gen, device=DEV).to(in_dt) for _ in range(W)]
    out = torch.randn(n, generator=gen, device=DEV).to(out_dt)
    into = to_np(out) if acc else None
    cp.cp_slot_sum(slots, out, accumulate=acc)
    ref = O.slot_sum([to_np(s) for s in slots], TAG[in_dt], TAG[out_dt], into=into)
    assert bits_equal(to_np(out), ref)


def test_slot_sum_just_under_the_threshold(cp):
    n = PIECE_MIN // 4 - 4
    say(f"case slot sum n={n} W=4 f32 (batched units)")
    gen = torch.Generator(device=DEV).manual_seed(3)
    slots = [torch.randn(n, generator=gen, device=DEV) for _ in range(4)]
    out = torch.empty(n, device=DEV)
    cp.cp_slot_sum(slots, out)
    assert bits_equal(to_np(out), O.slot_sum([to_np(s) for s in slots], "f32", "f32"))


# T = 32768 tokens of [16, 128]: with W = 4 every owner slot holds 8192 rows
# (32 MiB of bf16, 64 MiB of fp32) and every writer 32768 rows.
CU = {"dcs": np.array([0, 8192, 10240, 10240, 24576, 32768], np.int32),
      "pc": np.array([0, 1000, 1007, 1007, 21007, 32768], np.int32)}
POL = {"dcs": (0, O.DUAL_CHUNK_SWAP), "pc": (1, O.PACKED_CONTIGUOUS)}
GRAD_CASES = [(F32, F32, 4, "dcs", False), (F32, F32, 4, "pc", True), (F32, F32, 2, "dcs", True),
              (F32, BF16, 4, "dcs", True), (F32, BF16, 4, "pc", False),
              (BF16, BF16, 4, "dcs", False), (BF16, BF16, 4, "pc", True), (BF16, BF16, 2, "pc", False),
              (BF16, F32, 4, "dcs", True)]


@pytest.mark.parametrize("in_dt,out_dt,W,pol,acc", GRAD_CASES)
def test_grad_return_pieces(cp, in_dt, out_dt, W, pol, acc):
    """Unfused (scatter, owner sums) and fused gradient return of one [32768, 16, 128]
    tensor per writer: every slot and output element against the oracle."""
    T, H, D = 32768, 16, 128
    cu = CU[pol]
    say(f"case grad return pieces W={W} {pol} {in_dt}->{out_dt} accumulate={acc}")
    gen = torch.Generator(device=DEV).manual_seed(W + 100 * acc)
    grads = [[(torch.randn((T, H, D), generator=gen, device=DEV) * 1e-3).to(in_dt) for _ in range(W)]]
    into = [[torch.randn((T // W, H, D), generator=gen, device=DEV).to(out_dt) for _ in range(W)]]
    meta = cp.cp_build_meta(torch.from_numpy(cu).to(DEV), T, W, POL[pol][0], check=True)
    slots = [[[torch.empty((T // W, H, D), dtype=in_dt, device=DEV) for _ in range(W)] for _ in range(W)]]
    out = [[x.clone() for x in into[0]]]
    fused = [[x.clone() for x in into[0]]]
    cp.cp_grad_return(grads, slots, out, meta, accumulate=acc)
    cp.cp_grad_return_fused(grads, fused, meta, accumulate=acc)
    assert cp.cp_meta_status(meta)[0] == cp.CP_OK
    gn = [to_np(g) for g in grads[0]]
    iv = [to_np(x) for x in into[0]] if acc else None
    ref_slots, ref_out = O.grad_return(gn, cu, W, TAG[in_dt], TAG[out_dt], policy=POL[pol][1], into=iv)
    ref_fused = O.grad_return_fused(gn, cu, W, TAG[in_dt], TAG[out_dt], policy=POL[pol][1], into=iv)
    for o in range(W):
        for w in range(W):
            assert bits_equal(to_np(slots[0][o][w]), ref_slots[o][w]), (o, w)
        assert bits_equal(to_np(out[0][o]), ref_out[o]), o
        assert bits_equal(to_np(fused[0][o]), ref_fused[o]), o
    del grads, slots, out, fused
    torch.cuda.empty_cache()
