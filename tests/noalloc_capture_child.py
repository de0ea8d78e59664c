"""Child process of tests/test_zz_no_alloc.py: the first cp_grad_return_noalloc call of a
fresh process (so the one-time lookup of the static workspace's device address happens
then) is made under HIP graph capture; the replay must equal cp_grad_return run eagerly.
Prints one line, "first call captured ok" on success."""
import os
import sys

import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from thd_token_layout_amd import cpthd as cp  # noqa: E402

DEV = "cuda:0"
W, H, D, T = 4, 4, 128, 256
n = T // W
cu = torch.tensor([0, 64, 64, 192, 256], dtype=torch.int32, device=DEV)
meta = cp.cp_build_meta(cu, T, W, cp.CP_POLICY_DUAL_CHUNK_SWAP, check=True)
gen = torch.Generator(device=DEV).manual_seed(11)
grads = [[torch.randn((T, H, D), generator=gen, device=DEV) for _ in range(W)] for _ in range(2)]
got = [[torch.full((n, H, D), float("nan"), device=DEV) for _ in range(W)] for _ in range(2)]
ref = [[torch.empty((n, H, D), device=DEV) for _ in range(W)] for _ in range(2)]
slots = [[[torch.empty((n, H, D), device=DEV) for _ in range(W)] for _ in range(W)] for _ in range(2)]
torch.cuda.synchronize()
graph = torch.cuda.CUDAGraph()
with torch.cuda.graph(graph):
    cp.cp_grad_return_noalloc(grads, got, meta)
graph.replay()
cp.cp_grad_return(grads, slots, ref, meta)
torch.cuda.synchronize()
ok = all(torch.equal(got[t][o].view(torch.int32), ref[t][o].view(torch.int32)) for t in range(2) for o in range(W))
print("first call captured ok" if ok else "first call captured MISMATCH", flush=True)
