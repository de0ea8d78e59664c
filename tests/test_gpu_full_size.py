"""GPU parity at the full benchmark shapes, every element against the CPU oracle.

* The multi-tensor layout calls exactly as the benchmark makes them: Q, K, V
  [262144, 20, 128] bf16 through cp_partition_thd_multi / cp_gather_thd_multi
  for the packed-document dual-chunk-swap, packed-contiguous and one-document
  workloads (each tensor moves 2.7 GB, so the library launches once per tensor).
  Every element of every tensor is compared with the oracle's partition and
  gather.
* The W = 4 fp32 owner gradient return at S = 262144 and the W = 8 bf16 fused
  gradient return at S = 131072 ("Add stream-ordered CP gradient return
  primitive", section "Validation": the whole-tensor comparison at the
  S=262144 shape).  The writers' gradients are copied to the host once; then,
  one owner at a time, the oracle builds that owner's W slots and its sum from
  the host copies, and every slot, the unfused output and the fused output of
  that owner are compared in full.
"""
import numpy as np
import pytest
import torch

from gpu_util import DEV, O, WL, policy_name, say, to_np

pytestmark = pytest.mark.gpu

TAG = {torch.float32: "f32", torch.bfloat16: "bf16"}


@pytest.fixture(scope="module")
def cp():
    from thd_token_layout_amd import cpthd
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return cpthd


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what) -> None:
    """Bit-for-bit equality of two large arrays, compared in 64 MiB pieces."""
    assert got.shape == want.shape and got.dtype == want.dtype, (what, got.shape, want.shape)
    a = np.ascontiguousarray(got).reshape(-1).view(np.uint8)
    b = np.ascontiguousarray(want).reshape(-1).view(np.uint8)
    step = 64 << 20
    for k in range(0, a.size, step):
        if not np.array_equal(a[k:k + step], b[k:k + step]):
            bad = k + int(np.flatnonzero(a[k:k + step] != b[k:k + step])[0])
            row_bytes = a.size // got.shape[0] if got.shape and got.shape[0] else 1
            raise AssertionError(f"{what}: first differing byte {bad} (row {bad // row_bytes})")


def launches(cp, fn):
    """Run fn with the library's launch record on; return {kernel name: launches}."""
    torch.cuda.synchronize()
    cp.cp_profile_enable(True)
    fn()
    prof = cp.cp_profile_read()
    cp.cp_profile_enable(False)
    return {k: c for k, (c, _) in prof.items()}


# ------------------------------------------------------------------ layouts at S=262144
@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["dcs_s256k_w4", "pc_s256k_w4", "dcs1_s256k_w4"])
def test_multi_tensor_layout_full_compare(cp, name):
    w = WL.WORKLOADS[name]
    say(f"case {name}: multi-tensor partition + gather of Q, K, V, every element")
    cu = WL.cu_seqlens(w)
    pol = cp.POLICY[w.policy]
    W, T = w.cp_size, w.total_tokens
    meta = cp.cp_build_meta(torch.from_numpy(cu).to(DEV), T, W, pol, check=True)
    xs = WL.random_tensors(w, w.n_tensors, device=DEV)
    parts = [torch.empty((W, T // W, w.heads, w.head_dim), dtype=x.dtype, device=DEV) for x in xs]
    backs = [torch.empty_like(x) for x in xs]
    rec = launches(cp, lambda: cp.cp_partition_thd_multi(xs, meta, parts=parts))
    # each tensor moves >= 1 GiB, so the call runs one launch per tensor
    assert sum(rec.values()) == len(xs), rec
    rec = launches(cp, lambda: cp.cp_gather_thd_multi(parts, meta, xs=backs))
    assert sum(rec.values()) == len(xs), rec
    torch.cuda.synchronize()
    assert cp.cp_meta_status(meta)[0] == cp.CP_OK
    for k in range(len(xs)):
        xn = to_np(xs[k])
        ref = O.partition(xn, cu, W, policy_name(pol))
        got = to_np(parts[k])
        assert_bits_equal(got, ref, (name, "partition", k))
        del ref
        assert_bits_equal(to_np(backs[k]), O.gather(got, cu, W, policy_name(pol)), (name, "gather", k))
        del got, xn
    del xs, parts, backs
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ gradient return, per owner
class GradCase:
    """One gradient-return workload run on the GPU once (unfused with epochs, and
    fused), with host copies of every writer's gradients for the oracle."""

    def __init__(self, cp, name):
        w = WL.WORKLOADS[name]
        self.w = w
        self.W, self.T = w.cp_size, w.total_tokens
        W, n = self.W, self.T // self.W
        self.cu = WL.cu_seqlens(w)
        say(f"setup {name}: gradients, unfused and fused gradient return on the GPU")
        vals = WL.random_tensors(w, 2 * W, device=DEV)
        grads = [vals[:W], vals[W:]]  # dK, dV of writers 0..W-1
        self.in_dt = grads[0][0].dtype
        self.out_dt = torch.float32 if w.out_dtype == "f32" else torch.bfloat16
        meta = cp.cp_build_meta(torch.from_numpy(self.cu).to(DEV), self.T, W,
                                cp.CP_POLICY_DUAL_CHUNK_SWAP, check=True)
        shape = (n, w.heads, w.head_dim)
        self.slots = [[[torch.empty(shape, dtype=self.in_dt, device=DEV) for _ in range(W)] for _ in range(W)]
                      for _ in range(2)]
        self.out = [[torch.empty(shape, dtype=self.out_dt, device=DEV) for _ in range(W)] for _ in range(2)]
        self.fused = [[torch.empty(shape, dtype=self.out_dt, device=DEV) for _ in range(W)] for _ in range(2)]
        epochs = torch.zeros((W, W), dtype=torch.int32, device=DEV)
        cp.cp_grad_return(grads, self.slots, self.out, meta, epochs=epochs, epoch=1)
        cp.cp_grad_return_fused(grads, self.fused, meta)
        st = cp.cp_meta_status(meta)
        assert st[0] == cp.CP_OK, st
        assert (epochs == 1).all()
        self.host = [[to_np(g) for g in gt] for gt in grads]
        del vals, grads
        torch.cuda.empty_cache()

    def check_owner(self, t, o):
        W = self.W
        slots, out = O.grad_return(self.host[t], self.cu, W, TAG[self.in_dt], TAG[self.out_dt], owners=[o])
        for w in range(W):
            assert_bits_equal(to_np(self.slots[t][o][w]), slots[o][w], ("slot", t, o, w))
        assert_bits_equal(to_np(self.out[t][o]), out[o], ("out", t, o))
        assert_bits_equal(to_np(self.fused[t][o]), out[o], ("fused", t, o))


@pytest.fixture(scope="module")
def grad_s256k(cp):
    case = GradCase(cp, "grad_s256k_w4")
    yield case
    del case
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("t", [0, 1], ids=["dK", "dV"])
@pytest.mark.parametrize("o", range(4))
def test_grad_return_s256k_w4_every_element(grad_s256k, t, o):
    say(f"case grad_s256k_w4 tensor {t} owner {o}: 4 slots, unfused and fused output")
    grad_s256k.check_owner(t, o)


@pytest.fixture(scope="module")
def fused_s128k(cp):
    case = GradCase(cp, "fused_s128k_w8")
    yield case
    del case
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("t", [0, 1], ids=["dK", "dV"])
@pytest.mark.parametrize("o", range(8))
def test_fused_s128k_w8_every_element(fused_s128k, t, o):
    say(f"case fused_s128k_w8 tensor {t} owner {o}: 8 slots, unfused and fused output")
    fused_s128k.check_owner(t, o)
