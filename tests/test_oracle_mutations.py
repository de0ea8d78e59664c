"""Plant plausible mistakes in a private copy of the CPU oracle and check that the
pins catch every one of them (a dropped term, a wrong index, a transposed
operand, a reversed order, a wrong rounding)."""
import importlib.util
import os

import numpy as np
import pytest

import pins

ORACLE_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                           "oracle", "cp_oracle.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("cp_oracle_mutant", ORACLE_PATH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _dcs_swapped_chunks(o):
    def dcs_rank_rows(cu, cp_size, rank):
        W = cp_size
        pieces = [np.zeros(0, dtype=np.int64)]
        for b in range(len(cu) - 1):
            chunks = np.split(np.arange(int(cu[b]), int(cu[b + 1])), 2 * W)
            pieces += [chunks[2 * W - 1 - rank], chunks[rank]]
        return np.concatenate(pieces)
    return dcs_rank_rows


def _dcs_wrong_mirror(o):
    def dcs_rank_rows(cu, cp_size, rank):
        W = cp_size
        pieces = [np.zeros(0, dtype=np.int64)]
        for b in range(len(cu) - 1):
            chunks = np.split(np.arange(int(cu[b]), int(cu[b + 1])), 2 * W)
            pieces += [chunks[rank], chunks[W + rank]]
        return np.concatenate(pieces)
    return dcs_rank_rows


def _pc_keep_empty(o):
    orig = o.local_cu_seqlens

    def local_cu_seqlens(cu, total_tokens, cp_size, policy):
        if policy != o.PACKED_CONTIGUOUS:
            return orig(cu, total_tokens, cp_size, policy)
        W, B = cp_size, len(cu) - 1
        n = total_tokens // W
        local = np.zeros((W, B + 1), dtype=np.int32)
        n_local = np.zeros(W, dtype=np.int32)
        for r in range(W):
            inner = [int(v) - r * n for v in cu if r * n < int(v) < (r + 1) * n]  # duplicates kept
            row = [0] + inner + [n]
            n_local[r] = len(row) - 1
            local[r] = (row + [n] * (B + 1))[:B + 1]
        return local, n_local
    return local_cu_seqlens


def _pc_pad_zero(o):
    orig = o.local_cu_seqlens

    def local_cu_seqlens(cu, total_tokens, cp_size, policy):
        local, n_local = orig(cu, total_tokens, cp_size, policy)
        if policy == o.PACKED_CONTIGUOUS:
            for r in range(cp_size):
                local[r, n_local[r] + 1:] = 0
        return local, n_local
    return local_cu_seqlens


def _dcs_local_cu_halved(o):
    orig = o.local_cu_seqlens

    def local_cu_seqlens(cu, total_tokens, cp_size, policy):
        local, n_local = orig(cu, total_tokens, cp_size, policy)
        if policy == o.DUAL_CHUNK_SWAP:
            local = (np.asarray(cu, dtype=np.int32)[None, :] // (2 * cp_size)).repeat(cp_size, 0)
        return local, n_local
    return local_cu_seqlens


def _sum_reversed(o):
    def slot_sum(slots, in_dtype, out_dtype, into=None):
        slots = list(slots) if into is None else [into] + list(slots)
        acc = o._widen(slots[-1], in_dtype).astype(np.float32, copy=True)
        for w in range(len(slots) - 2, -1, -1):
            acc = (acc + o._widen(slots[w], in_dtype)).astype(np.float32)
        return o._narrow(acc, out_dtype)
    return slot_sum


def _sum_zero_seed(o):
    def slot_sum(slots, in_dtype, out_dtype, into=None):
        acc = np.zeros(slots[0].shape, dtype=np.float32)
        if into is not None:
            acc = (acc + o._widen(into, out_dtype)).astype(np.float32)
        for s in slots:
            acc = (acc + o._widen(s, in_dtype)).astype(np.float32)
        return o._narrow(acc, out_dtype)
    return slot_sum


def _sum_drops_last(o):
    def slot_sum(slots, in_dtype, out_dtype, into=None):
        acc = o._widen(slots[0], in_dtype).astype(np.float32, copy=True)
        if into is not None:
            acc = (o._widen(into, out_dtype) + acc).astype(np.float32)
        for w in range(1, len(slots) - 1):
            acc = (acc + o._widen(slots[w], in_dtype)).astype(np.float32)
        return o._narrow(acc, out_dtype)
    return slot_sum


def _bf16_truncate(o):
    def f32_to_bf16_rne(f32):
        return (np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return f32_to_bf16_rne


def _bf16_half_up(o):
    def f32_to_bf16_rne(f32):
        f32 = np.ascontiguousarray(f32, dtype=np.float32)
        u = f32.view(np.uint32).astype(np.uint64)
        r = ((u + np.uint64(0x8000)) >> np.uint64(16)).astype(np.uint32)
        q = ((u >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint32)
        return np.where(np.isnan(f32), q, r).astype(np.uint16)
    return f32_to_bf16_rne


def _scatter_transposed(o):
    def grad_scatter(grads, cu, cp_size, policy=o.DUAL_CHUNK_SWAP, owners=None):
        W = cp_size
        T = grads[0].shape[0]
        slots = [[None] * W for _ in range(W)]
        for w in range(W):
            for own in (range(W) if owners is None else owners):
                slots[own][w] = grads[own][o.rank_rows(cu, T, W, policy, w)]
        return slots
    return grad_scatter


def _fused_reversed(o):
    def grad_return_fused(grads, cu, cp_size, in_dtype, out_dtype, policy=o.DUAL_CHUNK_SWAP, into=None,
                          owners=None):
        W = cp_size
        T = grads[0].shape[0]
        out = [None] * W
        for own in (range(W) if owners is None else owners):
            rows = o.rank_rows(cu, T, W, policy, own)
            acc = o._widen(grads[W - 1][rows], in_dtype).astype(np.float32, copy=True)
            for w in range(W - 2, -1, -1):
                acc = (acc + o._widen(grads[w][rows], in_dtype)).astype(np.float32)
            if into is not None:
                acc = (acc + o._widen(into[own], out_dtype)).astype(np.float32)
            out[own] = o._narrow(acc, out_dtype)
        return out
    return grad_return_fused


def _no_decreasing_check(o):
    orig = o.cu_violations

    def cu_violations(cu, total_tokens, cp_size, policy):
        return orig(cu, total_tokens, cp_size, policy) - {"decreasing"}
    return cu_violations


def _pc_off_by_one(o):
    def pc_rank_rows(total_tokens, cp_size, rank):
        n = total_tokens // cp_size
        return (np.arange(rank * n, (rank + 1) * n, dtype=np.int64) + 1) % max(total_tokens, 1)
    return pc_rank_rows


def _acc_added_once(o):
    orig = o.slot_sum

    def slot_sum(slots, in_dtype, out_dtype, into=None):
        if into is None:
            return orig(slots, in_dtype, out_dtype)
        total = orig(slots, in_dtype, "f32")
        acc = (o._widen(into, out_dtype) + total).astype(np.float32)
        return o._narrow(acc, out_dtype)
    return slot_sum


def _acc_ignored(o):
    orig = o.grad_return_fused

    def grad_return_fused(grads, cu, cp_size, in_dtype, out_dtype, policy=o.DUAL_CHUNK_SWAP, into=None,
                          owners=None):
        return orig(grads, cu, cp_size, in_dtype, out_dtype, policy, owners=owners)
    return grad_return_fused


def _grad_policy_ignored(o):
    orig = o.grad_scatter

    def grad_scatter(grads, cu, cp_size, policy=o.DUAL_CHUNK_SWAP, owners=None):
        return orig(grads, cu, cp_size, o.DUAL_CHUNK_SWAP, owners)
    return grad_scatter


def _fused_policy_ignored(o):
    orig = o.grad_return_fused

    def grad_return_fused(grads, cu, cp_size, in_dtype, out_dtype, policy=o.DUAL_CHUNK_SWAP, into=None,
                          owners=None):
        return orig(grads, cu, cp_size, in_dtype, out_dtype, o.DUAL_CHUNK_SWAP, into, owners)
    return grad_return_fused


def _attn_kv_one_chunk_short(o):
    orig = o.attention_steps

    def attention_steps(cu, total_tokens, cp_size, policy, rank):
        steps = orig(cu, total_tokens, cp_size, policy, rank)
        if policy != o.DUAL_CHUNK_SWAP:
            return steps
        return [[(q0, ql, k0, kl - ql) for q0, ql, k0, kl in st] for st in steps]
    return attention_steps


def _attn_pc_no_lookback(o):
    orig = o.attention_steps

    def attention_steps(cu, total_tokens, cp_size, policy, rank):
        steps = orig(cu, total_tokens, cp_size, policy, rank)
        if policy != o.PACKED_CONTIGUOUS:
            return steps
        n = total_tokens // cp_size
        return [[(q0, ql, rank * n + q0, ql) for q0, ql, k0, kl in st] for st in steps]
    return attention_steps


def _attn_steps_swapped(o):
    orig = o.attention_steps

    def attention_steps(cu, total_tokens, cp_size, policy, rank):
        return orig(cu, total_tokens, cp_size, policy, rank)[::-1]
    return attention_steps


def _attn_offsets_packed(o):
    orig = o.attention_meta

    def attention_meta(cu, total_tokens, cp_size, policy):
        m = orig(cu, total_tokens, cp_size, policy)
        m["q_offsets"] = m["cu_seqlens_q"].copy()
        return m
    return attention_meta


def _ring_variant(o, direction=1, rs_shift=1, round_once=False, ag_steps=None):
    """A ring with one planted change: messages sent to rank r - 1 instead of
    r + 1, the wrong chunk index in the reduce-scatter, bf16 partials kept in
    fp32 until the end, or an all-gather step dropped."""
    def allreduce_ring(inputs, dtype):
        W = len(inputs)
        n = inputs[0].shape[0]
        ch = o.ring_chunks(n, W)
        wide = [o.bf16_to_f32(x) if dtype == "bf16" else x.copy() for x in inputs]
        buf = [x.copy() for x in wide]
        for s in range(W - 1):
            msgs = []
            for r in range(W):
                a, b = ch[(r - direction * (rs_shift + s)) % W]
                msgs.append((r, a, b, buf[(r - direction) % W][a:b].copy()))
            for r, a, b, m in msgs:
                acc = (m + wide[r][a:b]).astype(np.float32)
                if dtype == "bf16" and not round_once:
                    acc = o.bf16_to_f32(o.f32_to_bf16_rne(acc))
                buf[r][a:b] = acc
        for s in range(W - 1 if ag_steps is None else ag_steps(W)):
            msgs = []
            for r in range(W):
                a, b = ch[(r - direction * s) % W]
                msgs.append((r, a, b, buf[(r - direction) % W][a:b].copy()))
            for r, a, b, m in msgs:
                buf[r][a:b] = m
        return [o.f32_to_bf16_rne(x) if dtype == "bf16" else x for x in buf]
    return allreduce_ring


def _ring_reversed(o):
    return _ring_variant(o, direction=-1)


def _ring_rs_chunk_shifted(o):
    return _ring_variant(o, rs_shift=0)


def _ring_bf16_rounds_once(o):
    return _ring_variant(o, round_once=True)


def _ring_short_allgather(o):
    return _ring_variant(o, ag_steps=lambda W: max(W - 2, 0))


def _ring_rank_order(o):
    def allreduce_ring(inputs, dtype):
        return o.allreduce_one_shot(inputs, dtype)
    return allreduce_ring


def _ring_chunks_floor(o):
    def ring_chunks(n, cp_size):  # q = floor(n / W), the last chunk takes the rest
        q = n // cp_size
        return [(k * q, (k + 1) * q if k < cp_size - 1 else n) for k in range(cp_size)]
    return ring_chunks


def _ring_chunks_aligned(o):
    def ring_chunks(n, cp_size):  # chunk length rounded up to 64 elements
        q = -(-n // (64 * cp_size)) * 64
        return [(min(k * q, n), min((k + 1) * q, n)) for k in range(cp_size)]
    return ring_chunks


def _ring_chunks_balanced(o):
    def ring_chunks(n, cp_size):  # the first n % W chunks one element longer
        q, rem = divmod(n, cp_size)
        bounds = [k * q + min(k, rem) for k in range(cp_size + 1)]
        return [(bounds[k], bounds[k + 1]) for k in range(cp_size)]
    return ring_chunks


def _two_shot_wrong_owner(o):
    def allreduce_two_shot(inputs, dtype):
        W = len(inputs)
        n = inputs[0].shape[0]
        ch = o.ring_chunks(n, W)
        out = [np.empty_like(inputs[0]) for _ in range(W)]
        for c, (a, b) in enumerate(ch):
            src = ch[(c + 1) % W]  # owner c reduces the next chunk's rows
            m = min(b - a, src[1] - src[0])
            red = o.slot_sum([x[src[0]:src[0] + m] for x in inputs], dtype, dtype)
            for r in range(W):
                out[r][a:b] = 0
                out[r][a:a + m] = red
        return out
    return allreduce_two_shot


def _two_shot_no_gather(o):
    def allreduce_two_shot(inputs, dtype):
        W = len(inputs)
        ch = o.ring_chunks(inputs[0].shape[0], W)
        out = [x.copy() for x in inputs]
        for c, (a, b) in enumerate(ch):
            out[c][a:b] = o.slot_sum([x[a:b] for x in inputs], dtype, dtype)  # owners only
        return out
    return allreduce_two_shot


def _one_shot_reversed(o):
    def allreduce_one_shot(inputs, dtype):
        res = o.slot_sum(inputs[::-1], dtype, dtype)
        return [res.copy() for _ in inputs]
    return allreduce_one_shot


MUTATIONS = {
    "dcs_swapped_chunks": ("dcs_rank_rows", _dcs_swapped_chunks),
    "dcs_wrong_mirror": ("dcs_rank_rows", _dcs_wrong_mirror),
    "pc_keep_empty_docs": ("local_cu_seqlens", _pc_keep_empty),
    "pc_pad_with_zero": ("local_cu_seqlens", _pc_pad_zero),
    "dcs_local_cu_halved": ("local_cu_seqlens", _dcs_local_cu_halved),
    "sum_reversed": ("slot_sum", _sum_reversed),
    "sum_zero_seed": ("slot_sum", _sum_zero_seed),
    "sum_drops_last_slot": ("slot_sum", _sum_drops_last),
    "bf16_truncate": ("f32_to_bf16_rne", _bf16_truncate),
    "bf16_round_half_up": ("f32_to_bf16_rne", _bf16_half_up),
    "scatter_transposed": ("grad_scatter", _scatter_transposed),
    "fused_reversed": ("grad_return_fused", _fused_reversed),
    "no_decreasing_check": ("cu_violations", _no_decreasing_check),
    "pc_off_by_one": ("pc_rank_rows", _pc_off_by_one),
    "accumulate_added_once": ("slot_sum", _acc_added_once),
    "accumulate_ignored": ("grad_return_fused", _acc_ignored),
    "grad_scatter_ignores_policy": ("grad_scatter", _grad_policy_ignored),
    "fused_ignores_policy": ("grad_return_fused", _fused_policy_ignored),
    "attention_kv_one_chunk_short": ("attention_steps", _attn_kv_one_chunk_short),
    "attention_pc_no_lookback": ("attention_steps", _attn_pc_no_lookback),
    "attention_steps_swapped": ("attention_steps", _attn_steps_swapped),
    "attention_offsets_packed": ("attention_meta", _attn_offsets_packed),
    "ring_reversed": ("allreduce_ring", _ring_reversed),
    "ring_rs_chunk_shifted": ("allreduce_ring", _ring_rs_chunk_shifted),
    "ring_bf16_rounds_once": ("allreduce_ring", _ring_bf16_rounds_once),
    "ring_short_allgather": ("allreduce_ring", _ring_short_allgather),
    "ring_in_rank_order": ("allreduce_ring", _ring_rank_order),
    "ring_chunks_floor": ("ring_chunks", _ring_chunks_floor),
    "ring_chunks_aligned": ("ring_chunks", _ring_chunks_aligned),
    "ring_chunks_balanced": ("ring_chunks", _ring_chunks_balanced),
    "one_shot_reversed": ("allreduce_one_shot", _one_shot_reversed),
    "two_shot_wrong_owner": ("allreduce_two_shot", _two_shot_wrong_owner),
    "two_shot_no_gather": ("allreduce_two_shot", _two_shot_no_gather),
}

INVARIANT_CASES = [
    (2, "dual_chunk_swap", [0, 4, 4, 16, 24]),
    (3, "packed_contiguous", [0, 5, 5, 17, 30]),
    (4, "packed_contiguous", [0, 3, 9, 9, 20, 24]),
]


def run_all_pins(o):
    failures = []
    for check in pins.ALL_CHECKS:
        try:
            check(o)
        except (AssertionError, ValueError, IndexError) as e:  # noqa: PERF203
            failures.append((check.__name__, repr(e)[:80]))
    for W, pol, cu in INVARIANT_CASES:
        cu = np.array(cu, dtype=np.int32)
        T = int(cu[-1])
        x = np.random.default_rng(T).standard_normal((T, 2, 2)).astype(np.float32)
        try:
            pins.check_invariants(o, cu, T, W, pol, x)
        except (AssertionError, ValueError, IndexError) as e:
            failures.append(("invariants", repr(e)[:80]))
    return failures


def test_unmutated_oracle_passes_all_pins():
    assert run_all_pins(fresh_oracle()) == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    o = fresh_oracle()
    attr, make = MUTATIONS[name]
    setattr(o, attr, make(o))
    failures = run_all_pins(o)
    assert failures, f"planted mistake {name} passed every pin"
