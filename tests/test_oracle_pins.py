"""The CPU oracle against facts fixed outside of it (hand-worked tables, closed
forms, brute force, torch's bf16 cast, invariants)."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import pins
from oracle import cp_oracle as o


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(o)


@st.composite
def dcs_case(draw):
    W = draw(st.sampled_from([1, 2, 3, 4, 8]))
    ks = draw(st.lists(st.integers(0, 4), min_size=0, max_size=6))
    lengths = [2 * W * k for k in ks]
    return W, lengths


@st.composite
def pc_case(draw):
    W = draw(st.sampled_from([1, 2, 3, 4, 8]))
    lengths = draw(st.lists(st.integers(0, 23), min_size=1, max_size=8))
    T = sum(lengths)
    pad = (-T) % W
    lengths[-1] += pad
    return W, lengths


def _x(T, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, 2, 3)).astype(np.float32)


@settings(max_examples=60, deadline=None, derandomize=True)
@given(dcs_case())
def test_invariants_dcs(case):
    W, lengths = case
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    pins.check_invariants(o, cu, T, W, o.DUAL_CHUNK_SWAP, _x(T, T))


@settings(max_examples=60, deadline=None, derandomize=True)
@given(pc_case())
def test_invariants_pc(case):
    W, lengths = case
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    pins.check_invariants(o, cu, T, W, o.PACKED_CONTIGUOUS, _x(T, T + 1))


@settings(max_examples=40, deadline=None, derandomize=True)
@given(dcs_case(), st.integers(0, 2**31 - 1))
def test_brute_force_random(case, seed):
    W, lengths = case
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    rows = pins.brute_owner_rows(cu, T, W) if T else [[] for _ in range(W)]
    for r in range(W):
        assert o.rank_rows(cu, T, W, o.DUAL_CHUNK_SWAP, r).tolist() == rows[r]


@settings(max_examples=40, deadline=None, derandomize=True)
@given(dcs_case())
def test_attention_pairs_dcs(case):
    W, lengths = case
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    pins.check_attention_pairs(o, cu, int(cu[-1]), W, o.DUAL_CHUNK_SWAP)


@settings(max_examples=40, deadline=None, derandomize=True)
@given(pc_case())
def test_attention_pairs_pc(case):
    W, lengths = case
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    pins.check_attention_pairs(o, cu, int(cu[-1]), W, o.PACKED_CONTIGUOUS)


@settings(max_examples=40, deadline=None, derandomize=True)
@given(st.integers(1, 8), st.integers(1, 50), st.integers(0, 2**31 - 1), st.booleans())
def test_accumulate_exact_integers(W, n, seed, bf16_out):
    """Small integers are exact in fp32 (and bf16 up to 256): accumulating slots into
    an existing gradient must give the plain integer sum, whatever the order."""
    rng = np.random.default_rng(seed)
    slots = [rng.integers(-20, 21, size=n).astype(np.float32) for _ in range(W)]
    into = rng.integers(-50, 51, size=n).astype(np.float32)
    want = into.astype(np.int64) + sum(x.astype(np.int64) for x in slots)
    if bf16_out:
        got = o.bf16_to_f32(o.slot_sum(slots, "f32", "bf16", into=o.f32_to_bf16_rne(into)))
    else:
        got = o.slot_sum(slots, "f32", "f32", into=into)
    assert (got == want.astype(np.float32)).all()


@settings(max_examples=40, deadline=None, derandomize=True)
@given(pc_case(), st.integers(0, 2**31 - 1))
def test_pc_grad_return_random(case, seed):
    """Packed-contiguous owners: every slot is the writer's contiguous slice and the
    integer-valued sums are exact, for random documents and cp sizes."""
    W, lengths = case
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    rng = np.random.default_rng(seed)
    grads = [rng.integers(-9, 10, size=(T, 2)).astype(np.float32) for _ in range(W)]
    slots, out = o.grad_return(grads, cu, W, "f32", "f32", policy=o.PACKED_CONTIGUOUS)
    n = T // W
    total = sum(g.astype(np.int64) for g in grads)
    for owner in range(W):
        for w in range(W):
            assert (slots[owner][w] == grads[w][owner * n:(owner + 1) * n]).all()
        assert (out[owner] == total[owner * n:(owner + 1) * n].astype(np.float32)).all()


def test_empty_input():
    cu = np.array([0], dtype=np.int32)
    for pol in o.POLICIES:
        x = np.zeros((0, 2, 3), dtype=np.float32)
        parts = o.partition(x, cu, 4, pol)
        assert parts.shape == (4, 0, 2, 3)
        local, n_local = o.local_cu_seqlens(cu, 0, 4, pol)
        assert local.shape == (4, 1) and (local == 0).all()


def test_epochs_after():
    e = o.epochs_after(4, 7)
    assert e.shape == (4, 4) and (e == 7).all()


def test_bf16_rne_exhaustive():
    """Every one of the 2^32 fp32 bit patterns through the oracle's bf16 rounding
    against torch's CPU cast, in 256 chunks of 2^24 spread over threads (numpy and
    torch release the GIL)."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    import torch

    step = 1 << 24

    def run(start):
        pins.check_bf16_rne_bits(o, np.arange(start, start + step, dtype=np.uint64).astype(np.uint32))

    threads = max(1, min(8, len(os.sched_getaffinity(0))))
    torch_threads = torch.get_num_threads()
    torch.set_num_threads(1)  # one torch thread per worker: no oversubscription
    try:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(run, range(0, 1 << 32, step)))
    finally:
        torch.set_num_threads(torch_threads)


def _compositions(total, parts_max=None):
    """Every ordered list of positive integers summing to `total`."""
    if total == 0:
        yield []
        return
    for first in range(1, total + 1):
        for rest in _compositions(total - first):
            yield [first] + rest


def test_exhaustive_small_layouts():
    """Every document split of every small T (packed-contiguous: T <= 9; dual-chunk-
    swap: up to 5 chunk-lengths per rank), for W = 1..4: partition invariants, the
    brute-force owners, and the attention pairs against the brute-force mask."""
    count = 0
    for W in (1, 2, 3, 4):
        for T in range(0, 10):
            if T % W:
                continue
            for lengths in _compositions(T):
                cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
                x = np.arange(T * 2, dtype=np.float32).reshape(T, 1, 2)
                pins.check_invariants(o, cu, T, W, o.PACKED_CONTIGUOUS, x)
                pins.check_attention_pairs(o, cu, T, W, o.PACKED_CONTIGUOUS)
                count += 1
        for units in range(0, 6):  # total length in multiples of 2W
            for chunks in _compositions(units):
                lengths = [2 * W * c for c in chunks]
                cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
                T = int(cu[-1])
                x = np.arange(T * 2, dtype=np.float32).reshape(T, 1, 2)
                pins.check_invariants(o, cu, T, W, o.DUAL_CHUNK_SWAP, x)
                pins.check_attention_pairs(o, cu, T, W, o.DUAL_CHUNK_SWAP)
                if T:
                    rows = pins.brute_owner_rows(cu, T, W)
                    for r in range(W):
                        assert o.rank_rows(cu, T, W, o.DUAL_CHUNK_SWAP, r).tolist() == rows[r]
                count += 1
    assert count > 500


@settings(max_examples=80, deadline=None, derandomize=True)
@given(st.integers(1, 9), st.integers(0, 3000), st.sampled_from(["f32", "bf16"]), st.integers(0, 2 ** 31))
def test_allreduce_random(W, n, dt, seed):
    """All-reduce invariants on random sizes: every rank ends with the same bits
    under every algorithm; the two-shot equals the one-shot (both sum each element
    in rank order); the ring equals the closed rotated-order sum per chunk;
    integer-valued data gives the exact sum under all three."""
    rng = np.random.default_rng(seed)
    xs = [rng.standard_normal(n).astype(np.float32) for _ in range(W)]
    data = xs if dt == "f32" else [o.f32_to_bf16_rne(x) for x in xs]
    one = o.allreduce_one_shot(data, dt)
    two = o.allreduce_two_shot(data, dt)
    ring = o.allreduce_ring(data, dt)
    for res in (one, two, ring):
        assert len(res) == W and all(r.tobytes() == res[0].tobytes() for r in res)
    assert two[0].tobytes() == one[0].tobytes()
    want = np.empty_like(data[0])
    for k, (a, b) in enumerate(o.ring_chunks(n, W)):
        acc = data[k][a:b]
        for j in range(1, W):
            x = data[(k + j) % W][a:b]
            acc = (acc + x).astype(np.float32) if dt == "f32" else \
                o.f32_to_bf16_rne(o.bf16_to_f32(acc) + o.bf16_to_f32(x))
        want[a:b] = acc
    assert ring[0].tobytes() == want.tobytes()
    ints = [rng.integers(-500, 500, size=n).astype(np.float32) for _ in range(W)]
    exact = np.sum([i.astype(np.float64) for i in ints], axis=0) if n else np.zeros(0)
    for fn in (o.allreduce_one_shot, o.allreduce_two_shot, o.allreduce_ring):
        assert np.array_equal(fn(ints, "f32")[0].astype(np.float64), exact)


@settings(max_examples=30, deadline=None, derandomize=True)
@given(dcs_case(), st.booleans(), st.integers(0, 2**31 - 1))
def test_owner_subsets_match_the_full_call(case, pc, seed):
    """The oracle's gradient functions restricted to some owners give exactly the
    full call's arrays for those owners (and None for the others): the full-size
    GPU checks compare one owner at a time through these restricted calls."""
    W, lengths = case
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    pol = o.PACKED_CONTIGUOUS if pc else o.DUAL_CHUNK_SWAP
    rng = np.random.default_rng(seed)
    grads = [rng.standard_normal((T, 2)).astype(np.float32) for _ in range(W)]
    into = [rng.standard_normal((T // W, 2)).astype(np.float32) for _ in range(W)]
    full_slots, full_out = o.grad_return(grads, cu, W, "f32", "bf16", policy=pol)
    full_fused = o.grad_return_fused(grads, cu, W, "f32", "f32", policy=pol, into=into)
    owners = sorted(set(rng.integers(0, W, size=2).tolist()))
    slots, out = o.grad_return(grads, cu, W, "f32", "bf16", policy=pol, owners=owners)
    fused = o.grad_return_fused(grads, cu, W, "f32", "f32", policy=pol, into=into, owners=owners)
    for own in range(W):
        if own in owners:
            assert all(slots[own][w].tobytes() == full_slots[own][w].tobytes() for w in range(W))
            assert out[own].tobytes() == full_out[own].tobytes()
            assert fused[own].tobytes() == full_fused[own].tobytes()
        else:
            assert out[own] is None and fused[own] is None and all(s is None for s in slots[own])
