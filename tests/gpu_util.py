"""Helpers shared by the GPU tests: tensor <-> numpy bit views, workload setup."""
import sys

import numpy as np
import torch

from oracle import cp_oracle as O
from thd_token_layout_amd import workloads as WL

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_np(t: torch.Tensor) -> np.ndarray:
    """Exact host copy: float32 -> float32, bfloat16 -> uint16 bit patterns."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def np_dtype_tag(t: torch.Tensor) -> str:
    return {torch.float32: "f32", torch.bfloat16: "bf16"}[t.dtype]


def policy_name(code: int) -> str:
    return O.DUAL_CHUNK_SWAP if code == 0 else O.PACKED_CONTIGUOUS


def bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    return a.shape == b.shape and a.tobytes() == b.tobytes()


def max_abs_f32(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.max(np.abs(a.astype(np.float64) - b.astype(np.float64)))) if a.size else 0.0
