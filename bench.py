"""Benchmark: the THD context-parallel layout + gradient-return hot path at S=262144.

One step = one pass of every stage of the path over one batch of synthetic
input already resident in HBM:
  * metadata for the three token layouts (cp_build_meta) and the attention-step
    tables of both layout policies (cp_build_attn_meta),
  * dual-chunk-swap partition + inverse gather of Q, K, V [262144, 20, 128] bf16
    (packed documents, log-uniform lengths in [256, 8192], W = 4),
  * packed-contiguous partition + inverse gather of the same Q, K, V
    (documents of U{1..4096} tokens, W = 4),
  * owner gradient return, W = 4: 4 writers x {dK, dV} [262144, 20, 128] fp32
    scattered into 4 x 4 owner slots (two-chunk layout), epochs published and
    awaited, slots summed in fixed order into each owner's dK/dV,
  * fused scatter+sum gradient return on the same gradients,
  * the W = 8 fp32 slot-sum sweep, 1 KiB .. 16 MiB per slot.

Prints one JSON line: whole-step algorithmic HBM bytes / step time in GB/s,
the roofline of the dominant kernel (HIP events on its launch stream over the
timed region) beside the ceiling a plain stream of the same read/write mix and
size reaches on this GPU, and the CPU oracle's rate on the same step, on one
core and on the host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, AMD public specification
METRIC = "HBM GB/s & % of peak: THD CP partition/gather + dK/dV grad-return, S=262144"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sweep_buffers(WL, torch, dev):
    """[(bytes per slot, 8 fp32 slots, output)] for 1 KiB ... 16 MiB per slot."""
    w_sw = WL.WORKLOADS["sweep_w8"]
    res = []
    for nbytes in WL.SWEEP_BYTES:
        k = nbytes // 4
        slots = WL.random_tensors(w_sw, 8, shape=(k,), device=dev, seed_offset=nbytes)
        res.append((nbytes, slots, torch.empty(k, device=dev)))
    return res


class Step:
    """Buffers and calls of one step; every op records its algorithmic bytes."""

    def __init__(self, cp, WL, torch, S: int, device: str):
        self.cp, self.torch = cp, torch
        dev = device
        self.ops = []  # (name, bytes, callable)
        w_dcs = WL.WORKLOADS["dcs_s256k_w4"]
        w_pc = WL.WORKLOADS["pc_s256k_w4"]
        w_gr = WL.WORKLOADS["grad_s256k_w4"]
        if S != w_dcs.total_tokens:
            w_dcs, w_pc, w_gr = (WL.scaled(w, total_tokens=S) for w in (w_dcs, w_pc, w_gr))
        self.S = S
        self.workloads = (w_dcs, w_pc, w_gr)
        W = w_dcs.cp_size
        H, D = w_dcs.heads, w_dcs.head_dim
        # ---- layout inputs: the same Q, K, V under both policies, each policy with the
        # document set of its own workload (dcs_s256k_w4: log-uniform lengths, multiples
        # of 8; pc_s256k_w4: U{1..4096}).  per_config() also runs both policies on one
        # document set, where the policy is the only difference.
        self.cu_np = (WL.cu_seqlens(w_dcs), WL.cu_seqlens(w_pc), WL.cu_seqlens(w_gr))
        cu_dcs, cu_pc, cu_gr = (torch.from_numpy(c).to(dev) for c in self.cu_np)
        self.num_docs = (cu_dcs.numel() - 1, cu_pc.numel() - 1)
        self.qkv = WL.random_tensors(w_dcs, 3, device=dev)
        self.parts = [torch.empty((W, S // W, H, D), dtype=torch.bfloat16, device=dev) for _ in range(3)]
        self.back = [torch.empty_like(x) for x in self.qkv]
        self.meta_dcs = cp.cp_build_meta(cu_dcs, S, W, cp.CP_POLICY_DUAL_CHUNK_SWAP, check=True)
        self.meta_pc = cp.cp_build_meta(cu_pc, S, W, cp.CP_POLICY_PACKED_CONTIGUOUS, check=True)
        self.meta_gr = cp.cp_build_meta(cu_gr, S, W, cp.CP_POLICY_DUAL_CHUNK_SWAP, check=True)
        row_bf16 = H * D * 2
        # ---- gradient return inputs
        Wg = w_gr.cp_size
        n = S // Wg
        vals = WL.random_tensors(w_gr, 2 * Wg, device=dev)
        self.grads = [vals[:Wg], vals[Wg:]]
        row_f32 = w_gr.heads * w_gr.head_dim * 4
        self.slots = [[[torch.empty((n, w_gr.heads, w_gr.head_dim), device=dev) for _ in range(Wg)]
                       for _ in range(Wg)] for _ in range(2)]
        self.out = [[torch.empty((n, w_gr.heads, w_gr.head_dim), device=dev) for _ in range(Wg)]
                    for _ in range(2)]
        self.fused = [[torch.empty_like(o) for o in row] for row in self.out]
        self.epochs = torch.zeros((Wg, Wg), dtype=torch.int32, device=dev)
        self.epoch = 0
        # ---- sweep
        self.sweep = sweep_buffers(WL, torch, dev)

        metas = [(cu_dcs, cp.CP_POLICY_DUAL_CHUNK_SWAP, self.meta_dcs),
                 (cu_pc, cp.CP_POLICY_PACKED_CONTIGUOUS, self.meta_pc),
                 (cu_gr, cp.CP_POLICY_DUAL_CHUNK_SWAP, self.meta_gr)]

        def build_metas():
            for cu, pol, m in metas:
                cp.cp_build_meta(cu, S, m.cp_size, pol, meta=m.buf)

        meta_bytes = sum(4 * (cu.numel()) + 4 * (cu.numel()) * (W + 1) + 4 * W for cu, _, _ in metas)
        self.ops.append(("build_meta x3", meta_bytes, build_metas))
        # attention-step tables of both layout policies (written bytes; < 20 KB)
        attn = [(m, cp.cp_build_attn_meta(m)) for m in (self.meta_dcs, self.meta_pc)]
        attn_bytes = sum(2 * m.cp_size * (32 + 16 * (m.num_docs + 1)) for m, _ in attn)
        self.ops.append(("build_attn_meta x2", attn_bytes,
                         lambda: [cp.cp_build_attn_meta(m, attn=a) for m, a in attn]))
        for pname, meta in (("dual_chunk_swap", self.meta_dcs), ("packed_contiguous", self.meta_pc)):
            self.ops.append((f"partition_{pname} QKV", 3 * 2 * S * row_bf16,
                             lambda meta=meta: cp.cp_partition_thd_multi(self.qkv, meta, parts=self.parts)))
            self.ops.append((f"gather_{pname} QKV", 3 * 2 * S * row_bf16,
                             lambda meta=meta: cp.cp_gather_thd_multi(self.parts, meta, xs=self.back)))

        def grad_return():
            self.epoch += 1
            cp.cp_grad_return(self.grads, self.slots, self.out, self.meta_gr, epochs=self.epochs,
                              epoch=self.epoch)

        self.ops.append(("grad_return dK,dV", 2 * (3 * Wg + 1) * S * row_f32, grad_return))
        self.ops.append(("grad_return_fused dK,dV", 2 * (Wg + 1) * S * row_f32,
                         lambda: cp.cp_grad_return_fused(self.grads, self.fused, self.meta_gr)))
        self.ops.append(("slot_sum sweep W=8 1KiB..16MiB", sum(9 * nb for nb, _, _ in self.sweep),
                         lambda: [cp.cp_slot_sum(s, o) for _, s, o in self.sweep]))
        # per-launch algorithmic bytes of each kernel, by the kernel's role in its op
        self.kernel_bytes = {
            "scatter": 2 * S * row_f32,                 # one writer, one tensor: read T rows, write T rows
            "owner_sum": (Wg + 1) * n * row_f32,        # one owner, one tensor: read W slots, write 1
            "fused": (Wg + 1) * S * row_f32,            # one tensor, all owners
        }
        # read/write mix of each kernel role: (inputs, bytes per input and of the output),
        # for the plain stream that bounds it
        self.kernel_mix = {
            "scatter": (1, S * row_f32),
            "owner_sum": (Wg, n * row_f32),
            "fused": (Wg, S * row_f32),
            "layout": (1, S * row_bf16),
        }

    @property
    def step_bytes(self) -> int:
        return sum(b for _, b, _ in self.ops)

    def run(self):
        for _, _, fn in self.ops:
            fn()


def attribute_kernels(step: Step, cp, torch):
    """Run each op once with timing hooks on and map kernel name -> bytes per launch;
    also returns each kernel's milliseconds in that pass (which kernel dominates)."""
    per_kernel = {}
    mix = {}
    ms = {}
    torch.cuda.synchronize()
    cp.cp_profile_enable(True)
    for name, nbytes, fn in step.ops:
        fn()
        prof = cp.cp_profile_read()
        for kname, (count, kms) in prof.items():
            ms[kname] = ms.get(kname, 0.0) + kms
            role = None
            if name.startswith("grad_return dK"):
                role = "scatter" if kname.startswith("permute") else \
                    "owner_sum" if kname.startswith("slot_sum") else None
                b = step.kernel_bytes[role] if role else 0
            elif name.startswith("grad_return_fused"):
                role = "fused"
                b = step.kernel_bytes["fused"]
            elif name.startswith(("partition", "gather")):
                b = nbytes / count  # Q, K, V: one launch each, or one launch for all three
                if count == 3:
                    role = "layout"
            elif name.startswith("slot_sum sweep"):
                b = nbytes / count
            else:
                b = 0
            per_kernel.setdefault(kname, []).append((count, b))
            if role is not None:
                mix[kname] = step.kernel_mix[role]
    cp.cp_profile_enable(False)
    # bytes per step per kernel name, launches per step, stream mix per kernel name
    return {k: sum(c * b for c, b in v) for k, v in per_kernel.items()}, \
        {k: sum(c for c, _ in v) for k, v in per_kernel.items()}, mix, ms


def counted_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter runs.

    None when there is no record for this kernel or when any source the record
    was measured with has changed since (the counters would then be stale).
    """
    import hashlib

    path = os.path.join(ROOT, "profiles", "traffic_s262144.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel") != kernel:
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return int(round(rec["traffic_bytes_per_launch"]))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_inputs(step, torch):
    """Host copies of the step's inputs for the CPU oracle (bf16 as uint16 bits)."""
    import numpy as np

    def bits(t):
        t = t.detach()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()

    return {"cu": step.cu_np, "qkv": [bits(x) for x in step.qkv],
            "grads": [[bits(g) for g in gt] for gt in step.grads],
            "sweep": [(nb, [bits(x) for x in slots]) for nb, slots, _ in step.sweep],
            "S": step.S, "W": step.workloads[0].cp_size, "Wg": step.workloads[2].cp_size,
            "row_bf16": step.workloads[0].heads * step.workloads[0].head_dim * 2,
            "row_f32": step.workloads[2].heads * step.workloads[2].head_dim * 4}


def cpu_baseline(h, step_bytes: int, threads: int):
    """The CPU oracle, as it stands, on the whole step over the same inputs as the GPU
    (S = 262144): metadata and attention-step tables, DCS and PC partition + gather of
    Q, K, V, unfused and fused dK/dV gradient return, the W=8 sweep.  Timed once on one
    thread and once with the work split over `threads` threads (numpy releases the GIL):
    the items are independent oracle calls, one per tensor and policy for the layouts,
    one per owner and tensor for the gradient returns (the oracle's owners= argument)."""
    import time as _time
    from concurrent.futures import ThreadPoolExecutor

    from oracle import cp_oracle as O

    S, W, Wg = h["S"], h["W"], h["Wg"]
    cu_dcs, cu_pc, cu_gr = h["cu"]
    items = []
    for cu, pol in ((cu_dcs, O.DUAL_CHUNK_SWAP), (cu_pc, O.PACKED_CONTIGUOUS)):
        items.append(lambda cu=cu, pol=pol: (O.local_cu_seqlens(cu, S, W, pol), O.attention_meta(cu, S, W, pol)))
        for x in h["qkv"]:
            items.append(lambda x=x, cu=cu, pol=pol: O.gather(O.partition(x, cu, W, pol), cu, W, pol))
    items.append(lambda: O.local_cu_seqlens(cu_gr, S, Wg, O.DUAL_CHUNK_SWAP))
    for gt in h["grads"]:
        for o in range(Wg):
            items.append(lambda gt=gt, o=o: O.grad_return(gt, cu_gr, Wg, "f32", "f32", owners=[o]))
            items.append(lambda gt=gt, o=o: O.grad_return_fused(gt, cu_gr, Wg, "f32", "f32", owners=[o]))
    for _, slots in h["sweep"]:
        items.append(lambda slots=slots: O.slot_sum(slots, "f32", "f32"))
    order = list(range(len(items)))
    res = {}
    for n_thr in (1, threads):
        t0 = _time.perf_counter()
        if n_thr == 1:
            for k in order:
                items[k]()
        else:
            with ThreadPoolExecutor(max_workers=n_thr) as ex:
                list(ex.map(lambda k: items[k](), order))
        res[n_thr] = _time.perf_counter() - t0
    one, many = res[1], res[threads]
    return {"value": round(step_bytes / many / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "value_1core": round(step_bytes / one / 1e9, 3), "seconds_1core": round(one, 2),
            "seconds_ncore": round(many, 2), "cpu_model": cpu_model(),
            "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"one pass of the whole step at S={S} (the GPU step's own inputs, copied to the host): "
                      f"metadata and attention-step tables, DCS and PC partition+gather of Q,K,V "
                      f"[{S},20,128] bf16, unfused and fused dK/dV gradient return W={Wg} [{S},20,128] fp32, "
                      f"W=8 fp32 sweep 1 KiB..16 MiB; {step_bytes / 1e9:.1f} GB algorithmic; numpy oracle "
                      f"timed on 1 thread ({one:.1f} s) and on {threads} threads ({many:.1f} s), "
                      f"work split into {len(items)} independent oracle calls"}


def load_roofline_lib():
    """libcpthd_roofline.so: plain streaming kernels under the library's schedule."""
    import ctypes

    path = os.path.join(ROOT, "thd_token_layout_amd", "libcpthd_roofline.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not built: run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    lib.cprl_stream.restype = ctypes.c_int
    lib.cprl_stream.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_int64,
                                ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    return lib


class Ceiling:
    """What a plain stream of a read/write mix reaches on this GPU: n_in inputs of
    `nbytes` each read and (write) one output of `nbytes` written, by the streaming
    kernels of libcpthd_roofline.so (full grid, contiguous tiles, 16-byte non-temporal
    loads, as the library's kernels), the best of 1, 2 and 3 units per thread (4, 8 and
    12 KiB tiles), of two load schedules (a thread's loads all in flight, or one at a
    time), with one unit per thread of 256- and 64-thread workgroups, and, when writing,
    of two store policies (non-temporal global stores; buffer stores with the nt and sc1
    cache policy).  With `launches` = k, k such streams on k sets of buffers launched back
    to back and timed together (the ceiling of an operation that makes k launches of that
    size).  Timed like per_config: median of `reps` runs per shape, each after a 1 GiB
    write that flushes the last-level cache, with HIP events on the stream the kernels
    are launched on.  Results are cached by mix, size and launch count."""

    def __init__(self, torch, dev, reps: int = 10):
        self.lib = load_roofline_lib()
        self.torch, self.dev, self.reps = torch, dev, reps
        self.cache = {}
        self.flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        self.sink = torch.zeros(1024, dtype=torch.int32, device=dev)

    def rate(self, n_in: int, nbytes: int, write: bool = True, launches: int = 1):
        import ctypes
        import statistics

        torch = self.torch
        nbytes = (int(nbytes) + 15) // 16 * 16
        key = (n_in, nbytes, write, launches)
        if key in self.cache:
            return self.cache[key]
        sets = []
        for _ in range(launches):
            ins = [torch.empty(nbytes, dtype=torch.uint8, device=self.dev) for _ in range(n_in)]
            out = torch.empty(nbytes, dtype=torch.uint8, device=self.dev) if write else None
            tab = (ctypes.c_void_p * max(n_in, 1))(*[t.data_ptr() for t in ins])
            outp = ctypes.c_void_p(out.data_ptr()) if write else None
            sets.append((ins, out, tab, outp))
        sink = ctypes.c_void_p(self.sink.data_ptr())

        def launch(shape):
            np_, pol, ser, small = shape
            stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for _, _, tab, outp in sets:
                st = self.lib.cprl_stream(n_in, tab, outp, nbytes, np_, sink,
                                          pol | (2 if ser else 0) | (4 if small else 0), stream)
                if st != 0:
                    raise RuntimeError(f"cprl_stream: status {st}")

        by_shape = {}
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # one load in flight differs from all in flight only with several loads per thread
        # 64-thread workgroups only with one unit per thread
        shapes = [(np_, pol, ser, small) for small in (0, 1) for ser in (0, 1) for pol in ((0, 1) if write else (0,))
                  for np_ in (1, 2, 3) if (not ser or np_ * n_in > 1) and (not small or np_ == 1)]
        for shape in shapes:
            launch(shape)
            ts = []
            for _ in range(self.reps):
                self.flush.fill_(1.0)
                e0.record()
                launch(shape)
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1000.0)
            by_shape[shape] = statistics.median(ts)
        best = min(by_shape, key=by_shape.get)
        us = by_shape[best]
        moved = nbytes * (n_in + (1 if write else 0)) * launches
        mix = f"{n_in}:{1 if write else 0}" if n_in else "0:1"
        policy = ("nt", "nt+sc1")
        loads = ("all in flight", "one in flight")
        res = {"mix": mix, "bytes_per_buffer": nbytes, "moved_bytes": moved, "median_us": round(us, 2),
               "gbs": round(moved / us / 1e3, 1), "units_per_thread": best[0], "stores": policy[best[1]],
               "loads": loads[best[2]], "threads_per_workgroup": 64 if best[3] else 256,
               "gbs_by_shape": {f"{k[0]} units/thread, {policy[k[1]]} stores, loads {loads[k[2]]}, "
                                f"{64 if k[3] else 256} threads": round(moved / v / 1e3, 1)
                                for k, v in by_shape.items()}}
        if launches > 1:
            res["launches"] = launches
        self.cache[key] = res
        del sets
        torch.cuda.empty_cache()
        return res

    def standard(self, S: int):
        """The mixes and sizes of the step's kernels at S tokens, plus pure read and write."""
        row_bf16, row_f32 = 20 * 128 * 2, 20 * 128 * 4
        return {
            "copy 1:1, one layout tensor (S x 5 KiB)": self.rate(1, S * row_bf16),
            "copy 1:1, one writer's gradient (S x 10 KiB; the scatter)": self.rate(1, S * row_f32),
            "4:1, four owner slots (S/4 x 10 KiB each; the owner sum)": self.rate(4, S // 4 * row_f32),
            "4:1, four writers' gradients (S x 10 KiB each; the fused sum)": self.rate(4, S * row_f32),
            "read only (S x 10 KiB)": self.rate(1, S * row_f32, write=False),
            "write only (S x 10 KiB)": self.rate(0, S * row_f32),
        }


def attn_summary(cp, meta):
    """Attention-step counts and sizes from the tables cp_build_attn_meta writes: steps per
    rank, segments over all ranks and steps, summed query and key rows, longest key range."""
    attn = cp.cp_build_attn_meta(meta)
    magic, t = cp.read_attn_meta(attn, meta.num_docs, meta.cp_size)
    if magic != cp.CP_ATTN_MAGIC:
        raise RuntimeError("attention tables were not built")
    seg = t["num_segments"]
    return {"steps_per_rank": int((seg > 0).sum(dim=1).max()), "segments": int(seg.sum()),
            "total_q": int(t["total_q"].sum()), "total_kv": int(t["total_kv"].sum()),
            "max_seqlen_kv": int(t["max_seqlen_kv"].max())}


def per_config(cp, WL, torch, dev, reps: int = 10, ceiling=None, names=None):
    """Each workload's ops timed on their own: median of `reps` HIP-event timings,
    each preceded by a 1 GiB write that flushes the 256 MB last-level cache.  With a
    Ceiling, each single-kernel row also gets the plain stream of the same read/write mix
    and size, and the row's fraction of it.  The dual-chunk-swap S=262144 workload is also
    run under packed-contiguous ownership with the same documents and the same Q, K, V
    (the policy the only difference), with each policy's attention-step tables summarised."""
    import statistics

    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    results = []

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts = []
        fn()  # warm
        for _ in range(reps):
            flush.fill_(1.0)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1000.0)
        return statistics.median(ts)

    def n_launches(fn):
        """Library launches one call of `fn` makes (its ceiling is that many plain streams)."""
        torch.cuda.synchronize()
        cp.cp_profile_enable(True)
        fn()
        prof = cp.cp_profile_read()
        cp.cp_profile_enable(False)
        return max(1, sum(c for c, _ in prof.values()))

    def add(cfg, op, nbytes, us, mix=None, **extra):
        row = {"config": cfg, "op": op, "bytes": nbytes, "median_us": round(us, 1),
               "gbs": round(nbytes / us / 1e3, 1), "frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
        if ceiling is not None and mix is not None and nbytes:
            c = ceiling.rate(*mix)
            row["ceiling_gbs"] = c["gbs"]
            row["frac_of_ceiling"] = round(row["gbs"] / c["gbs"], 4)
        row.update(extra)
        results.append(row)

    layout = ("dcs_t32k_w4", "pc_t64k_w4", "dcs_s256k_w4", "pc_s256k_w4", "dcs1_s256k_w4")
    for name in layout:
        if names and name not in names:
            continue
        w = WL.WORKLOADS[name]
        cu_np = WL.cu_seqlens(w)
        cu = torch.from_numpy(cu_np).to(dev)
        xs = WL.random_tensors(w, w.n_tensors, device=dev)
        parts = [torch.empty((w.cp_size, w.total_tokens // w.cp_size, w.heads, w.head_dim),
                             dtype=x.dtype, device=dev) for x in xs]
        back = [torch.empty_like(x) for x in xs]
        nbytes = sum(2 * x.numel() * x.element_size() for x in xs)
        policies = [(w.policy, cp.POLICY[w.policy])]
        if name == "dcs_s256k_w4":  # matched inputs: the same documents and tensors under both policies
            policies.append(("packed_contiguous", cp.CP_POLICY_PACKED_CONTIGUOUS))
        for pname, pol in policies:
            meta = cp.cp_build_meta(cu, w.total_tokens, w.cp_size, pol, check=True)
            cfg = name if pol == cp.POLICY[w.policy] else f"{name} as packed_contiguous (same documents and Q,K,V)"
            docs = {"documents": int(cu.numel() - 1), "attention": attn_summary(cp, meta)}
            # a ceiling of as many plain streams as the call makes launches (the multi-tensor
            # call launches once, or once per tensor when each tensor moves >= 1 GiB)
            part_multi = lambda: cp.cp_partition_thd_multi(xs, meta, parts=parts)
            gather_multi = lambda: cp.cp_gather_thd_multi(parts, meta, xs=back)
            part_single = lambda: [cp.cp_partition_thd(x, meta, parts=p) for x, p in zip(xs, parts)]
            for op, fn, kw in (("partition Q,K,V (multi-tensor call)", part_multi, docs),
                               ("gather Q,K,V (multi-tensor call)", gather_multi, {}),
                               ("partition Q,K,V (three single-tensor calls)", part_single, {})):
                k = n_launches(fn)
                add(cfg, op, nbytes, timed(fn), mix=(1, nbytes // 2 // k, True, k), **kw)
            add(cfg, "metadata", 0, timed(lambda: cp.cp_build_meta(cu, w.total_tokens, w.cp_size, pol,
                                                                     meta=meta.buf)))
            attn = cp.cp_build_attn_meta(meta)
            add(cfg, "attention-step metadata", 0, timed(lambda: cp.cp_build_attn_meta(meta, attn=attn)))
        del xs, parts, back
        torch.cuda.empty_cache()
    for name in ("grad_s256k_w4", "fused_s128k_w8"):
        if names and name not in names:
            continue
        w = WL.WORKLOADS[name]
        W, S = w.cp_size, w.total_tokens
        n = S // W
        cu = torch.from_numpy(WL.cu_seqlens(w)).to(dev)
        meta = cp.cp_build_meta(cu, S, W, cp.CP_POLICY_DUAL_CHUNK_SWAP, check=True)
        vals = WL.random_tensors(w, 2 * W, device=dev)
        grads = [vals[:W], vals[W:]]
        dt = grads[0][0].dtype
        row_in = w.heads * w.head_dim * grads[0][0].element_size()
        out = [[torch.empty((n, w.heads, w.head_dim), dtype=dt, device=dev) for _ in range(W)]
               for _ in range(2)]
        add(name, "fused grad return dK,dV", 2 * (W + 1) * S * row_in,
            timed(lambda: cp.cp_grad_return_fused(grads, out, meta)), mix=(W, S * row_in, True, 2))
        slots = [[[torch.empty((n, w.heads, w.head_dim), dtype=dt, device=dev) for _ in range(W)]
                  for _ in range(W)] for _ in range(2)]
        epochs = torch.zeros((W, W), dtype=torch.int32, device=dev)
        state = {"e": 0}

        def unfused():
            state["e"] += 1
            cp.cp_grad_return(grads, slots, out, meta, epochs=epochs, epoch=state["e"])

        add(name, "grad return dK,dV (scatter, epochs, owner sums)", 2 * (3 * W + 1) * S * row_in,
            timed(unfused))
        # accumulate mode: the owner's gradient is read as well (one more row per output row)
        add(name, "fused grad return dK,dV, accumulate", 2 * (W + 2) * S * row_in,
            timed(lambda: cp.cp_grad_return_fused(grads, out, meta, accumulate=True)), mix=(W + 1, S * row_in, True, 2))
        # the same tensors under packed-contiguous ownership (owner o: tokens [o S/W, (o+1) S/W))
        meta_pc = cp.cp_build_meta(cu, S, W, cp.CP_POLICY_PACKED_CONTIGUOUS, check=True)
        add(name, "fused grad return dK,dV, packed-contiguous owners", 2 * (W + 1) * S * row_in,
            timed(lambda: cp.cp_grad_return_fused(grads, out, meta_pc)), mix=(W, S * row_in, True, 2))

        def unfused_pc():
            state["e"] += 1
            cp.cp_grad_return(grads, slots, out, meta_pc, epochs=epochs, epoch=state["e"])

        add(name, "grad return dK,dV, packed-contiguous owners", 2 * (3 * W + 1) * S * row_in,
            timed(unfused_pc))
        del vals, grads, out, slots
        torch.cuda.empty_cache()
    del flush
    torch.cuda.empty_cache()
    return results


def graph_us_per_call(torch, fn, calls: int = 100, replays: int = 5):
    """`fn` captured `calls` times back to back in one HIP graph and replayed:
    per-call time without host work or per-launch submission."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(calls):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) * 1000.0 / (calls * replays)


def eager_us_per_call(torch, fn, reps: int):
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000.0 / reps


def c_abi_call(cp, torch, name, *args):
    """A call of the C entry point `name` with its arguments marshalled once (ctypes),
    on torch's current stream: the eager cost of the C ABI without the binding's
    per-call marshalling."""
    import ctypes

    fn = getattr(cp.lib, name)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = fn(*args, stream)
    if st != 0:
        raise RuntimeError(f"{name}: status {st}")
    return lambda: fn(*args, stream)


def kernel_us_per_call(cp, fn, calls: int = 20):
    """Summed duration of the kernels one call launches (HIP events around each launch)."""
    cp.cp_profile_enable(True)
    for _ in range(calls):
        fn()
    prof = cp.cp_profile_read()
    cp.cp_profile_enable(False)
    return sum(m for _, m in prof.values()) * 1000.0 / calls, sum(c for c, _ in prof.values()) // calls


def sweep_latency(step: Step, cp, torch, reps: int = 1000):
    """Per-call latency of the W=8 slot sum: eager through the Python binding (marshalling +
    host validation + launch + kernel), eager through the C ABI with arguments marshalled
    once, the kernel alone (HIP events around each launch), and replayed from a HIP graph."""
    res = []
    import ctypes

    res = []
    for nbytes, slots, out in step.sweep:
        def call():
            cp.cp_slot_sum(slots, out)
        raw = c_abi_call(cp, torch, "cp_slot_sum", len(slots),
                         (ctypes.c_void_p * len(slots))(*[t.data_ptr() for t in slots]),
                         ctypes.c_void_p(out.data_ptr()), out.numel(), cp.CP_F32, cp.CP_F32, 0)
        kus, _ = kernel_us_per_call(cp, call)
        res.append({"bytes_per_slot": nbytes, "us_per_call": round(eager_us_per_call(torch, call, reps), 2),
                    "c_abi_us_per_call": round(eager_us_per_call(torch, raw, reps), 2),
                    "kernel_us": round(kus, 2),
                    "graph_us_per_call": round(graph_us_per_call(torch, call), 2)})
    return res


def allreduce_sweep(sweep, cp, torch):
    """All-reduce of W=8 fp32 rank buffers of 1 KiB ... 16 MiB, every rank emulated on this
    GPU: one-shot (one launch, each rank reads all 8 buffers) against ring (14 launches:
    7 reduce-scatter and 7 all-gather steps), two-shot (2 launches) and the ring in one
    launch with in-kernel signals.  Per call: eager latency (through the binding and through the
    C ABI), summed kernel time, and (launch-per-step forms) time replayed from a HIP graph;
    algorithmic bytes over all 8 ranks (one-shot 72 x size, ring 35 x size, two-shot
    23 x size) over the kernel time."""
    import ctypes

    W = 8
    res = []
    for nbytes, slots, _ in sweep:
        outs = [torch.empty_like(slots[0]) for _ in range(W)]
        row = {"bytes_per_rank": nbytes}
        for algo, factor in (("one_shot", W * (W + 1)), ("ring", 5 * (W - 1)), ("two_shot", 3 * W - 1)):
            def call(algo=algo):
                cp.cp_allreduce(slots, outs, algo=algo)
            raw = c_abi_call(cp, torch, "cp_allreduce", cp.ALLREDUCE_ALGOS[algo], W,
                             (ctypes.c_void_p * W)(*[t.data_ptr() for t in slots]),
                             (ctypes.c_void_p * W)(*[t.data_ptr() for t in outs]), slots[0].numel(), cp.CP_F32)
            kus, launches = kernel_us_per_call(cp, call)
            row[algo] = {"us_per_call": round(eager_us_per_call(torch, call, 200), 2),
                         "c_abi_us_per_call": round(eager_us_per_call(torch, raw, 200), 2),
                         "kernel_us": round(kus, 2), "launches": launches,
                         "graph_us_per_call": round(graph_us_per_call(torch, call, calls=20), 2),
                         "kernel_gbs": round(factor * nbytes / (kus * 1e-6) / 1e9, 1) if kus > 0 else None}
        # the ring in one launch (in-kernel signals): every call needs a new epoch, so it
        # is timed eagerly only (a captured call would replay a stale epoch)
        sig = torch.zeros(cp.cp_allreduce_signal_bytes(W), dtype=torch.uint8, device=slots[0].device)
        epoch = [0]

        def call_sig():
            epoch[0] += 1
            cp.cp_allreduce_signal(slots, sig, epoch[0], outs=outs)

        fn = cp.lib.cp_allreduce_signal
        tin = (ctypes.c_void_p * W)(*[t.data_ptr() for t in slots])
        tout = (ctypes.c_void_p * W)(*[t.data_ptr() for t in outs])
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

        def raw_sig():
            epoch[0] += 1
            fn(W, tin, tout, slots[0].numel(), cp.CP_F32, ctypes.c_void_p(sig.data_ptr()), sig.numel(),
               epoch[0], 0, stream)

        kus, launches = kernel_us_per_call(cp, call_sig)
        row["ring_one_launch"] = {"us_per_call": round(eager_us_per_call(torch, call_sig, 200), 2),
                                  "c_abi_us_per_call": round(eager_us_per_call(torch, raw_sig, 200), 2),
                                  "kernel_us": round(kus, 2), "launches": launches,
                                  "kernel_gbs": round(5 * (W - 1) * nbytes / (kus * 1e-6) / 1e9, 1) if kus > 0 else None}
        if cp.cp_allreduce_signal_status(sig, W, epoch[0]) != cp.CP_OK:
            raise RuntimeError("one-launch ring reported a stale epoch or a timeout")
        res.append(row)
        del outs, sig
    faster = [r["bytes_per_rank"] for r in res
              if r["ring"]["graph_us_per_call"] < r["one_shot"]["graph_us_per_call"]]
    best = {r["bytes_per_rank"]: min(("one_shot", "ring", "two_shot"), key=lambda k: r[k]["graph_us_per_call"])
            for r in res}
    return {"cp_size": W, "dtype": "f32", "sizes": res,
            "ring_faster_from_bytes": min(faster) if faster else None,
            "fastest_graph_replayed": best}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--tokens", type=int, default=262144, help="S (default 262144)")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="threads of the CPU oracle's N-core run (default: the usable host CPUs, at most 16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the plain-stream ceiling measurements")
    ap.add_argument("--only-ceiling", action="store_true",
                    help="run only the plain-stream ceilings of the step's mixes and print them as one JSON "
                         "line (for profiling them on their own; not the benchmark line)")
    ap.add_argument("--config-names", default="",
                    help="comma-separated workloads for --only-configs (default: all)")
    ap.add_argument("--no-sweep-latency", action="store_true")
    ap.add_argument("--no-allreduce", action="store_true",
                    help="skip the one-shot / ring all-reduce sweep")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload measurements (each config's ops timed alone)")
    ap.add_argument("--only-configs", action="store_true",
                    help="run only the per-workload measurements and print them as one JSON line "
                         "(for profiling them on their own; not the benchmark line)")
    ap.add_argument("--only-allreduce", action="store_true",
                    help="run only the one-shot / ring all-reduce sweep and print it as one JSON line "
                         "(for profiling it on its own; not the benchmark line)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="run one plain 1 GiB device copy (torch copy_) first, as the reference "
                         "dispatch for scaling hardware traffic counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the W context-parallel ranks are emulated as slot "
              "buffers in one GPU's HBM, and no multi-GPU path is built; run with --gpus 1.",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch

    from thd_token_layout_amd import cpthd as cp
    from thd_token_layout_amd import workloads as WL

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.calibration_copy:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log("[bench] calibration copy: 1 GiB read + 1 GiB written")
        del a, b
    if args.only_allreduce:
        log("[bench] all-reduce sweep only")
        print(json.dumps({"allreduce_sweep": allreduce_sweep(sweep_buffers(WL, torch, dev), cp, torch)}),
              flush=True)
        return
    if args.only_configs:
        log("[bench] per-config measurements only")
        names = [n for n in args.config_names.split(",") if n] or None
        ceil = None if args.no_ceiling else Ceiling(torch, dev)
        print(json.dumps({"per_config": per_config(cp, WL, torch, dev, ceiling=ceil, names=names)}), flush=True)
        return
    if args.only_ceiling:
        log("[bench] plain-stream ceilings only")
        print(json.dumps({"ceiling": Ceiling(torch, dev).standard(args.tokens)}), flush=True)
        return
    log(f"[bench] building inputs S={args.tokens}")
    step = Step(cp, WL, torch, args.tokens, dev)
    torch.cuda.synchronize()
    log("[bench] attributing kernels")
    kbytes, kcount, kmix, kms = attribute_kernels(step, cp, torch)
    dominant = max(kms, key=kms.get)  # the kernel with the most time in one pass
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()

    # The timed steps record events around the dominant kernel's launches only:
    # an event pair around every launch would add about 0.5 ms of GPU time per
    # step (two event records per launch, about 55 launches).
    log(f"[bench] timing {args.steps} steps (HIP events around {dominant})")
    cp.cp_profile_select(dominant)
    cp.cp_profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step.run()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    cp.cp_profile_enable(False)
    cp.cp_profile_select(None)
    prof_dom = cp.cp_profile_read(capacity=256)
    ms_per_step = (t1 - t0) * 1000.0 / args.steps
    step_bytes = step.step_bytes
    value = step_bytes / (ms_per_step / 1000.0) / 1e9
    log(f"[bench] {ms_per_step:.3f} ms/step, {value:.1f} GB/s")
    # every kernel's time, from two more steps with events around every launch
    prof_steps = 2
    cp.cp_profile_enable(True)
    for _ in range(prof_steps):
        step.run()
    torch.cuda.synchronize()
    cp.cp_profile_enable(False)
    prof_all = cp.cp_profile_read(capacity=256)

    def kernel_row(name, count, total_ms, steps, where):
        b = kbytes.get(name, 0) * steps
        return {"kernel": name, "launches": count, "avg_us": round(total_ms * 1000 / count, 2),
                "total_ms": round(total_ms, 3),
                "gbs": round(b / (total_ms / 1000.0) / 1e9, 1) if total_ms > 0 and b else None,
                "bytes_per_launch": int(b / count) if count else 0, "timed": where}

    kernels = [kernel_row(n, c, t, prof_steps, "profiled steps after the timed region")
               for n, (c, t) in prof_all.items() if n != dominant]
    kernels.sort(key=lambda k: -k["total_ms"])
    c, t = prof_dom[dominant]
    dom = kernel_row(dominant, c, t, args.steps, "timed region")
    kernels.insert(0, dom)
    achieved = dom["gbs"] or 0.0
    traffic = counted_traffic(dom["kernel"])
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled "
                                "by a 1 GiB copy; profiles/traffic_s262144.md)",
                "kernel": dom["kernel"], "bytes_per_launch": dom["bytes_per_launch"],
                "avg_launch_us": dom["avg_us"]}

    sweep = None if args.no_sweep_latency else sweep_latency(step, cp, torch)
    if not args.no_allreduce:
        log("[bench] all-reduce sweep (one-shot, ring)")
    allreduce = None if args.no_allreduce else allreduce_sweep(step.sweep, cp, torch)
    num_docs = step.num_docs
    ops = [{"op": n, "bytes": b} for n, b, _ in step.ops]
    host = None
    if not args.no_cpu_baseline:
        log("[bench] copying the step's inputs to the host for the CPU oracle")
        host = host_inputs(step, torch)
    del step  # free the step's buffers (~70 GB) before the ceiling and per-workload runs
    torch.cuda.empty_cache()
    ceiling = None
    if not args.no_ceiling:
        log("[bench] plain-stream ceilings")
        ceil = Ceiling(torch, dev)
        ceiling = ceil.standard(args.tokens)
        for k in kernels:
            if k["kernel"] in kmix:
                c = ceil.rate(*kmix[k["kernel"]])
                k["ceiling_mix"] = c["mix"]
                k["ceiling_gbs"] = c["gbs"]
                if k["gbs"]:
                    k["frac_of_ceiling"] = round(k["gbs"] / c["gbs"], 4)
        if dom["kernel"] in kmix:
            c = ceil.rate(*kmix[dom["kernel"]])
            roofline["ceiling"] = {"mix": c["mix"], "gbs": c["gbs"], "bytes_per_buffer": c["bytes_per_buffer"],
                                   "what": "a plain stream of the same read/write mix and size under the same "
                                           "schedule (libcpthd_roofline.so), HIP-event median of 10"}
            roofline["frac_of_ceiling"] = round(achieved / c["gbs"], 4) if achieved else None
    configs = None
    if not args.no_configs:
        log("[bench] per-config measurements")
        configs = per_config(cp, WL, torch, dev, ceiling=None if args.no_ceiling else ceil)
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"THD CP layout + gradient return at S={args.tokens}: DCS and packed-contiguous "
                        f"partition+gather of Q,K,V [S,20,128] bf16 (W=4), dK/dV gradient return "
                        f"unfused and fused (W=4, [S,20,128] fp32), W=8 fp32 slot-sum sweep",
            "S": args.tokens, "cp_size": 4, "heads": 20, "head_dim": 128,
            "layout_dtype": "bf16", "grad_dtype": "f32", "accumulate": "f32",
            "docs_dcs": num_docs[0], "docs_pc": num_docs[1],
            "step_bytes": step_bytes,
        },
        "roofline": roofline,
        "kernels": kernels,
        "ops": ops,
        "sweep_latency": sweep,
        "allreduce_sweep": allreduce,
        "per_config": configs,
        "ceiling": ceiling,
        "device": torch.cuda.get_device_name(0),
    }
    if host is not None:
        threads = args.cpu_threads or min(16, len(os.sched_getaffinity(0)))
        log(f"[bench] CPU oracle baseline at S={args.tokens}, 1 thread and {threads} threads")
        result["cpu_baseline"] = cpu_baseline(host, step_bytes, threads)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
