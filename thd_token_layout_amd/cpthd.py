"""Python binding of libcpthd (C ABI in include/cpthd.h).

Argument marshalling only: torch tensors are turned into device pointers and
the current HIP stream, the C entry point of the same name is called (ctypes
releases the GIL during the call), and a non-zero status raises CpError.  Every
step of the computation runs in the HIP kernels of libcpthd.so; importing this
module raises ImportError when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcpthd.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"libcpthd.so not found at {_LIB_PATH}: build it with "
        "`python -m thd_token_layout_amd.build` (hipcc, gfx950)")
lib = ctypes.CDLL(_LIB_PATH)
LIB_PATH = _LIB_PATH

# ---------------------------------------------------------------- constants (cpthd.h)
CP_OK, CP_ERR_ARG, CP_ERR_UNSUPPORTED, CP_ERR_SHAPE, CP_ERR_DEVICE = 0, 1, 2, 3, 4
CP_ERR_ALIAS, CP_ERR_HIP, CP_ERR_TIMEOUT, CP_ERR_META, CP_ERR_TOO_LARGE = 5, 6, 7, 8, 9
CP_POLICY_DUAL_CHUNK_SWAP, CP_POLICY_PACKED_CONTIGUOUS = 0, 1
CP_F32, CP_BF16, CP_F16, CP_FP8_E4M3, CP_FP8_E5M2 = 0, 1, 2, 3, 4
CP_ALL_RANKS = -1
CP_MAX_CP_SIZE = 64
CP_PHASE_SCATTER, CP_PHASE_PUBLISH, CP_PHASE_WAIT, CP_PHASE_SUM = 0x1, 0x2, 0x4, 0x8
CP_PHASE_ALL = 0xF
CP_SUM_ACCUMULATE = 0x10
CP_NOALLOC_SCRATCH_BYTES = 64 << 20
CP_META_MAGIC = 0x48545043
CP_META_FIRST_NOT_ZERO = 0x0001
CP_META_DECREASING = 0x0002
CP_META_LAST_NOT_TOTAL = 0x0004
CP_META_DOC_NOT_DIVISIBLE = 0x0008
CP_META_BUILD_MASK = 0x00FF
CP_CALL_BAD_MAGIC = 0x0100
CP_CALL_TOKENS_MISMATCH = 0x0200
CP_CALL_CP_SIZE_MISMATCH = 0x0400
CP_CALL_POLICY_MISMATCH = 0x0800
CP_CALL_USED_INVALID_META = 0x1000
CP_CALL_DOCS_MISMATCH = 0x2000
CP_ATTN_MAGIC = 0x54414350
CP_ALLREDUCE_ONE_SHOT, CP_ALLREDUCE_RING, CP_ALLREDUCE_TWO_SHOT = 0, 1, 2

POLICY = {"dual_chunk_swap": CP_POLICY_DUAL_CHUNK_SWAP,
          "packed_contiguous": CP_POLICY_PACKED_CONTIGUOUS}

_c = ctypes
_vp = _c.c_void_p
_i32, _i64, _u32, _u64, _sz = _c.c_int32, _c.c_int64, _c.c_uint32, _c.c_uint64, _c.c_size_t

lib.cp_meta_bytes.restype = _sz
lib.cp_meta_bytes.argtypes = [_i32, _i32]
lib.cp_meta_bytes_row_maps.restype = _sz
lib.cp_meta_bytes_row_maps.argtypes = [_i32, _i32, _i64]
lib.cp_build_meta.restype = _c.c_int
lib.cp_build_meta.argtypes = [_vp, _i32, _i64, _i32, _i32, _vp, _sz, _vp]
lib.cp_meta_status.restype = _c.c_int
lib.cp_meta_status.argtypes = [_vp, _vp, _c.POINTER(_i32), _c.POINTER(_u64)]
lib.cp_partition_thd.restype = _c.c_int
lib.cp_partition_thd.argtypes = [_vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp]
lib.cp_gather_thd.restype = _c.c_int
lib.cp_gather_thd.argtypes = [_vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp]
lib.cp_partition_thd_multi.restype = _c.c_int
lib.cp_partition_thd_multi.argtypes = [_i32, _c.POINTER(_vp), _c.POINTER(_vp), _i64, _i32, _i32, _i32,
                                       _vp, _vp]
lib.cp_gather_thd_multi.restype = _c.c_int
lib.cp_gather_thd_multi.argtypes = [_i32, _c.POINTER(_vp), _c.POINTER(_vp), _i64, _i32, _i32, _i32,
                                    _vp, _vp]
lib.cp_grad_return.restype = _c.c_int
lib.cp_grad_return.argtypes = [_i32, _i32, _i32, _c.POINTER(_vp), _c.POINTER(_vp), _c.POINTER(_vp),
                               _i64, _i32, _i32, _i32, _i32, _vp, _vp, _u32, _i64, _i32, _vp]
lib.cp_grad_return_noalloc.restype = _c.c_int
lib.cp_grad_return_noalloc.argtypes = [_i32, _i32, _c.POINTER(_vp), _c.POINTER(_vp), _i64, _i32, _i32, _i32,
                                       _i32, _vp, _i32, _vp]
lib.cp_grad_return_fused.restype = _c.c_int
lib.cp_grad_return_fused.argtypes = [_i32, _i32, _i32, _c.POINTER(_vp), _c.POINTER(_vp), _i64, _i32,
                                     _i32, _i32, _i32, _vp, _i32, _vp]
lib.cp_slot_sum.restype = _c.c_int
lib.cp_slot_sum.argtypes = [_i32, _c.POINTER(_vp), _vp, _i64, _i32, _i32, _i32, _vp]
lib.cp_allreduce.restype = _c.c_int
lib.cp_allreduce.argtypes = [_i32, _i32, _c.POINTER(_vp), _c.POINTER(_vp), _i64, _i32, _vp]
lib.cp_allreduce_signal_bytes.restype = _sz
lib.cp_allreduce_signal_bytes.argtypes = [_i32]
lib.cp_allreduce_signal.restype = _c.c_int
lib.cp_allreduce_signal.argtypes = [_i32, _c.POINTER(_vp), _c.POINTER(_vp), _i64, _i32, _vp, _sz, _u64,
                                    _i64, _vp]
lib.cp_allreduce_signal_status.restype = _c.c_int
lib.cp_allreduce_signal_status.argtypes = [_vp, _i32, _u64, _vp]
lib.cp_attn_meta_bytes.restype = _sz
lib.cp_attn_meta_bytes.argtypes = [_i32, _i32]
lib.cp_build_attn_meta.restype = _c.c_int
lib.cp_build_attn_meta.argtypes = [_vp, _i32, _i32, _vp, _sz, _vp]
lib.cp_status_string.restype = _c.c_char_p
lib.cp_status_string.argtypes = [_c.c_int]
lib.cp_version.restype = _c.c_int
lib.cp_version.argtypes = []
lib.cp_profile_enable.restype = _c.c_int
lib.cp_profile_enable.argtypes = [_c.c_int]
lib.cp_profile_select.restype = _c.c_int
lib.cp_profile_select.argtypes = [_c.c_char_p]
lib.cp_profile_read.restype = _c.c_int
lib.cp_profile_read.argtypes = [_c.c_char_p, _c.POINTER(_i64), _c.POINTER(_c.c_double), _c.c_int]


class CpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {cp_status_string(status)} (status {status})")


def _check(status: int, where: str) -> None:
    if status != CP_OK:
        raise CpError(status, where)


def cp_status_string(status: int) -> str:
    return lib.cp_status_string(int(status)).decode()


def cp_version() -> int:
    return lib.cp_version()


_DTYPES = {torch.float32: CP_F32, torch.bfloat16: CP_BF16, torch.float16: CP_F16}
for _name, _code in (("float8_e4m3fn", CP_FP8_E4M3), ("float8_e5m2", CP_FP8_E5M2)):
    if hasattr(torch, _name):
        _DTYPES[getattr(torch, _name)] = _code


def dtype_code(dt: torch.dtype) -> int:
    try:
        return _DTYPES[dt]
    except KeyError:
        raise TypeError(f"unsupported dtype {dt}") from None


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, like: Optional[torch.Tensor] = None) -> int:
    """The HIP stream handle: `stream` if given, else torch's current stream."""
    if stream is None:
        if _raw_stream is not None:
            dev = like.device.index if like is not None and like.device.index is not None \
                else torch.cuda.current_device()
            return _raw_stream(dev)
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if t.numel() == 0:
        return t.data_ptr() or None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libcpthd must be contiguous")
    return t.data_ptr()


def _table(rows) -> "ctypes.Array":
    flat = [_ptr(t) for t in rows]
    return (_vp * len(flat))(*flat)


@dataclass
class Meta:
    """Device metadata buffer plus the host-side parameters it was built from."""
    buf: torch.Tensor        # uint8 device tensor of cp_meta_bytes(B, W) bytes
    cp_size: int
    policy: int
    num_docs: int
    total_tokens: int

    @property
    def local_tokens(self) -> int:
        return self.total_tokens // self.cp_size

    def ptr(self) -> int:
        return self.buf.data_ptr()


def cp_meta_bytes(num_docs: int, cp_size: int) -> int:
    return lib.cp_meta_bytes(num_docs, cp_size)


def cp_meta_bytes_row_maps(num_docs: int, cp_size: int, total_tokens: int) -> int:
    return lib.cp_meta_bytes_row_maps(num_docs, cp_size, total_tokens)


def cp_build_meta(cu_seqlens: torch.Tensor, total_tokens: int, cp_size: int, policy,
                  meta: Optional[torch.Tensor] = None, stream=None, check: bool = False,
                  row_maps: bool = True) -> Meta:
    """Validate cu_seqlens on the device and build per-rank metadata.

    A new buffer holds the row maps too under dual-chunk-swap (row_maps=True).
    With check=True the stream is synchronized and a data error raises CpError.
    """
    if isinstance(policy, str):
        policy = POLICY[policy]
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    B = cu_seqlens.numel() - 1
    nbytes = cp_meta_bytes(B, cp_size)
    if row_maps and policy == CP_POLICY_DUAL_CHUNK_SWAP and total_tokens > 0:
        nbytes = cp_meta_bytes_row_maps(B, cp_size, int(total_tokens)) or nbytes
    if meta is None:
        meta = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=cu_seqlens.device)
    st = lib.cp_build_meta(_ptr(cu_seqlens), B, int(total_tokens), int(cp_size), int(policy),
                           _ptr(meta), meta.numel(), _stream(stream, cu_seqlens))
    _check(st, "cp_build_meta")
    m = Meta(meta, int(cp_size), int(policy), B, int(total_tokens))
    if check:
        status, flags, _ = cp_meta_status(m, stream)
        if status != CP_OK:
            raise CpError(status, f"cp_build_meta: invalid cu_seqlens (flags 0x{flags:x})")
    return m


def cp_meta_status(meta, stream=None):
    """Synchronize and return (status, flags, wait_timeout_ranks)."""
    buf = meta.buf if isinstance(meta, Meta) else meta
    flags = _i32(0)
    timeouts = _u64(0)
    st = lib.cp_meta_status(_ptr(buf), _stream(stream, buf), ctypes.byref(flags), ctypes.byref(timeouts))
    if st not in (CP_OK, CP_ERR_META, CP_ERR_TIMEOUT):
        raise CpError(st, "cp_meta_status")
    return st, flags.value, timeouts.value


def read_local_cu(meta: Meta):
    """(local_cu [W, B+1], n_local [W]) copied from the device metadata (synchronizes)."""
    B, W = meta.num_docs, meta.cp_size
    words = meta.buf[: 64 + 4 * (B + 1) * (W + 1) + 4 * W].cpu().view(torch.int32)
    base = 16 + (B + 1)
    local = words[base: base + W * (B + 1)].reshape(W, B + 1).clone()
    n_local = words[base + W * (B + 1): base + W * (B + 1) + W].clone()
    return local, n_local


def read_row_maps(meta: Meta):
    """(row_of_local [T], local_of_row [T]) int32 copied from the device metadata, or None
    when it was built without them (synchronizes)."""
    header = meta.buf[:64].cpu().view(torch.int32)
    if int(header[12]) != 1:  # cp_meta_header.row_maps (byte offset 48)
        return None
    T = meta.total_tokens
    off = cp_meta_bytes(meta.num_docs, meta.cp_size)
    words = meta.buf[off: off + 8 * T].cpu().view(torch.int32)
    return words[:T].clone(), words[T:].clone()


def cp_attn_meta_bytes(num_docs: int, cp_size: int) -> int:
    return lib.cp_attn_meta_bytes(num_docs, cp_size)


def cp_build_attn_meta(meta: Meta, attn: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Per-rank attention-step tables (uint8 device buffer) from built metadata."""
    nbytes = cp_attn_meta_bytes(meta.num_docs, meta.cp_size)
    if attn is None:
        attn = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=meta.buf.device)
    st = lib.cp_build_attn_meta(meta.ptr(), meta.num_docs, meta.cp_size, _ptr(attn), attn.numel(),
                                _stream(stream, meta.buf))
    _check(st, "cp_build_attn_meta")
    return attn


ATTN_SCALARS = ("num_segments", "max_seqlen_q", "max_seqlen_kv", "total_q", "total_kv")
ATTN_TABLES = ("cu_seqlens_q", "cu_seqlens_kv", "q_offsets", "kv_offsets")


def read_attn_meta(attn: torch.Tensor, num_docs: int, cp_size: int):
    """Copy the attention-step tables to the host (synchronizes): (magic, dict of int32
    tensors [W, 2] for the scalars and [W, 2, B+1] for the tables)."""
    B, W = num_docs, cp_size
    rec = 8 + 4 * (B + 1)  # int32 words per step record
    words = attn[: 64 + 4 * 2 * W * rec].cpu().view(torch.int32)
    magic = int(words[0].item()) & 0xFFFFFFFF
    recs = words[16: 16 + 2 * W * rec].reshape(W, 2, rec)
    out = {k: recs[:, :, i].clone() for i, k in enumerate(ATTN_SCALARS)}
    for i, k in enumerate(ATTN_TABLES):
        out[k] = recs[:, :, 8 + i * (B + 1): 8 + (i + 1) * (B + 1)].clone()
    return magic, out


def cp_partition_thd(x: torch.Tensor, meta: Meta, parts: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    T, H, D = x.shape
    if parts is None:
        parts = torch.empty((meta.cp_size, T // meta.cp_size, H, D), dtype=x.dtype, device=x.device)
    st = lib.cp_partition_thd(_ptr(x), _ptr(parts), T, H, D, dtype_code(x.dtype), meta.ptr(),
                              _stream(stream, x))
    _check(st, "cp_partition_thd")
    return parts


def cp_gather_thd(parts: torch.Tensor, meta: Meta, x: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    W, n, H, D = parts.shape
    T = W * n
    if x is None:
        x = torch.empty((T, H, D), dtype=parts.dtype, device=parts.device)
    st = lib.cp_gather_thd(_ptr(parts), _ptr(x), T, H, D, dtype_code(parts.dtype), meta.ptr(),
                           _stream(stream, parts))
    _check(st, "cp_gather_thd")
    return x


def cp_partition_thd_multi(xs: Sequence[torch.Tensor], meta: Meta,
                           parts: Optional[Sequence[torch.Tensor]] = None, stream=None):
    """Partition several tensors of one shape (e.g. Q, K, V) in one launch."""
    T, H, D = xs[0].shape
    if parts is None:
        parts = [torch.empty((meta.cp_size, T // meta.cp_size, H, D), dtype=x.dtype, device=x.device)
                 for x in xs]
    st = lib.cp_partition_thd_multi(len(xs), _table(xs), _table(parts), T, H, D, dtype_code(xs[0].dtype),
                                    meta.ptr(), _stream(stream, xs[0]))
    _check(st, "cp_partition_thd_multi")
    return list(parts)


def cp_gather_thd_multi(parts: Sequence[torch.Tensor], meta: Meta,
                        xs: Optional[Sequence[torch.Tensor]] = None, stream=None):
    """Inverse of cp_partition_thd_multi."""
    W, n, H, D = parts[0].shape
    T = W * n
    if xs is None:
        xs = [torch.empty((T, H, D), dtype=p.dtype, device=p.device) for p in parts]
    st = lib.cp_gather_thd_multi(len(parts), _table(parts), _table(xs), T, H, D,
                                 dtype_code(parts[0].dtype), meta.ptr(), _stream(stream, parts[0]))
    _check(st, "cp_gather_thd_multi")
    return list(xs)


def _flat2(tab: Sequence[Sequence[Optional[torch.Tensor]]]):
    return [t for row in tab for t in row]


def _flat3(tab):
    return [t for a in tab for b in a for t in b]


def cp_grad_return(grads: Sequence[Sequence[torch.Tensor]], slots, out, meta: Meta,
                   rank: int = CP_ALL_RANKS, epochs: Optional[torch.Tensor] = None,
                   epoch: int = 0, wait_timeout_us: int = 0, phases: int = CP_PHASE_ALL,
                   accumulate: bool = False, stream=None) -> None:
    """grads[t][w] [T,H,D]; slots[t][o][w] [T/W,H,D]; out[t][o] [T/W,H,D] (overwritten, or
    accumulated into when `accumulate`)."""
    n_tensors = len(grads)
    W = len(grads[0])
    ref = next(g for g in _flat2(grads) if g is not None)
    T, H, D = ref.shape
    out_ref = next(o for o in _flat2(out) if o is not None)
    st = lib.cp_grad_return(int(rank), W, n_tensors, _table(_flat2(grads)), _table(_flat3(slots)),
                            _table(_flat2(out)), T, H, D, dtype_code(ref.dtype),
                            dtype_code(out_ref.dtype), meta.ptr(), _ptr(epochs), int(epoch),
                            int(wait_timeout_us), int(phases) | (CP_SUM_ACCUMULATE if accumulate else 0),
                            _stream(stream, ref))
    _check(st, "cp_grad_return")


def cp_grad_return_fused(grads, out, meta: Meta, rank: int = CP_ALL_RANKS, accumulate: bool = False,
                         stream=None) -> None:
    n_tensors = len(grads)
    W = len(grads[0])
    ref = next(g for g in _flat2(grads) if g is not None)
    T, H, D = ref.shape
    out_ref = next(o for o in _flat2(out) if o is not None)
    st = lib.cp_grad_return_fused(int(rank), W, n_tensors, _table(_flat2(grads)), _table(_flat2(out)),
                                  T, H, D, dtype_code(ref.dtype), dtype_code(out_ref.dtype),
                                  meta.ptr(), CP_SUM_ACCUMULATE if accumulate else 0, _stream(stream, ref))
    _check(st, "cp_grad_return_fused")


def cp_grad_return_noalloc(grads, out, meta: Meta, accumulate: bool = False, stream=None) -> None:
    """cp_grad_return for every rank in stream order with the owner slots in the library's
    static device workspace: grads[t][w] [T,H,D], out[t][o] [T/W,H,D]."""
    n_tensors = len(grads)
    W = len(grads[0])
    T, H, D = grads[0][0].shape
    st = lib.cp_grad_return_noalloc(W, n_tensors, _table(_flat2(grads)), _table(_flat2(out)), T, H, D,
                                    dtype_code(grads[0][0].dtype), dtype_code(out[0][0].dtype), meta.ptr(),
                                    CP_SUM_ACCUMULATE if accumulate else 0, _stream(stream, grads[0][0]))
    _check(st, "cp_grad_return_noalloc")


def cp_slot_sum(slots: Sequence[torch.Tensor], out: torch.Tensor, accumulate: bool = False,
                stream=None) -> torch.Tensor:
    st = lib.cp_slot_sum(len(slots), _table(slots), _ptr(out), out.numel(),
                         dtype_code(slots[0].dtype), dtype_code(out.dtype),
                         CP_SUM_ACCUMULATE if accumulate else 0, _stream(stream, out))
    _check(st, "cp_slot_sum")
    return out


ALLREDUCE_ALGOS = {"one_shot": CP_ALLREDUCE_ONE_SHOT, "ring": CP_ALLREDUCE_RING,
                   "two_shot": CP_ALLREDUCE_TWO_SHOT}


def _uniform_table(ts, dtype, n: int) -> "ctypes.Array":
    """Pointer table of contiguous tensors that all have `dtype` and `n` elements."""
    ptrs = []
    for t in ts:
        if t.dtype != dtype or t.numel() != n or not t.is_contiguous():
            raise ValueError("cp_allreduce: W contiguous inputs and W outputs of one dtype and size")
        ptrs.append(t.data_ptr() or None)
    return (_vp * len(ptrs))(*ptrs)


def cp_allreduce(inputs: Sequence[torch.Tensor], outs: Optional[Sequence[torch.Tensor]] = None,
                 algo: str = "one_shot", stream=None) -> List[torch.Tensor]:
    """Every rank's out = the sum of all W inputs (W rank buffers on this device)."""
    if outs is None:
        outs = [torch.empty_like(x) for x in inputs]
    if len(outs) != len(inputs):
        raise ValueError("cp_allreduce: as many outputs as inputs")
    x0 = inputs[0]
    dt, n = x0.dtype, x0.numel()
    st = lib.cp_allreduce(ALLREDUCE_ALGOS[algo], len(inputs), _uniform_table(inputs, dt, n),
                          _uniform_table(outs, dt, n), n, dtype_code(dt), _stream(stream, x0))
    _check(st, "cp_allreduce")
    return list(outs)


def cp_allreduce_signal_bytes(cp_size: int) -> int:
    return lib.cp_allreduce_signal_bytes(cp_size)


def cp_allreduce_signal(inputs: Sequence[torch.Tensor], signals: torch.Tensor, epoch: int,
                        outs: Optional[Sequence[torch.Tensor]] = None, wait_timeout_us: int = 0,
                        stream=None) -> List[torch.Tensor]:
    """The ring all-reduce in one launch, ranks signalling each hop through `signals`
    (a zero-filled device buffer of cp_allreduce_signal_bytes(W) bytes; `epoch` must
    exceed that of every earlier call on it)."""
    if outs is None:
        outs = [torch.empty_like(x) for x in inputs]
    if len(outs) != len(inputs):
        raise ValueError("cp_allreduce_signal: as many outputs as inputs")
    x0 = inputs[0]
    dt, n = x0.dtype, x0.numel()
    st = lib.cp_allreduce_signal(len(inputs), _uniform_table(inputs, dt, n), _uniform_table(outs, dt, n), n,
                                 dtype_code(dt), _ptr(signals), signals.numel() * signals.element_size(),
                                 int(epoch), int(wait_timeout_us), _stream(stream, x0))
    _check(st, "cp_allreduce_signal")
    return list(outs)


def cp_allreduce_signal_status(signals: torch.Tensor, cp_size: int, epoch: int, stream=None) -> int:
    """Synchronize, then CP_OK / CP_ERR_ARG (stale epoch) / CP_ERR_TIMEOUT for the call of `epoch`."""
    return lib.cp_allreduce_signal_status(_ptr(signals), cp_size, int(epoch), _stream(stream, signals))


def cp_profile_enable(enable: bool = True) -> None:
    _check(lib.cp_profile_enable(1 if enable else 0), "cp_profile_enable")


def cp_profile_select(name: Optional[str] = None) -> None:
    """Record only the kernel reported under `name` (None: every kernel)."""
    _check(lib.cp_profile_select(name.encode() if name else None), "cp_profile_select")


def cp_profile_read(capacity: int = 64):
    """{kernel name: (launches, total ms)} recorded since the last read (synchronizes)."""
    names = ctypes.create_string_buffer(128 * capacity)
    counts = (_i64 * capacity)()
    ms = (ctypes.c_double * capacity)()
    k = lib.cp_profile_read(names, counts, ms, capacity)
    if k < 0:
        raise CpError(-k, "cp_profile_read")
    res = {}
    for i in range(min(k, capacity)):
        nm = names.raw[128 * i: 128 * (i + 1)].split(b"\0", 1)[0].decode()
        res[nm] = (int(counts[i]), float(ms[i]))
    return res


EXPORTED = ["cp_meta_bytes", "cp_meta_bytes_row_maps", "cp_build_meta", "cp_meta_status", "cp_attn_meta_bytes", "cp_build_attn_meta",
            "cp_partition_thd", "cp_gather_thd",
            "cp_partition_thd_multi", "cp_gather_thd_multi",
            "cp_grad_return", "cp_grad_return_noalloc", "cp_grad_return_fused", "cp_slot_sum", "cp_allreduce",
            "cp_allreduce_signal_bytes", "cp_allreduce_signal", "cp_allreduce_signal_status",
            "cp_status_string", "cp_version",
            "cp_profile_enable", "cp_profile_select", "cp_profile_read"]
