"""Checks that pin the CPU oracle to facts fixed outside of it.

Each check takes the oracle module as its argument so the same check can be run
against a deliberately broken copy (see test_oracle_mutations.py) to show it
catches that mistake.  None of these checks retypes an oracle formula: they use
hand-worked tables from the pages' rules (tests/golden), closed forms,
brute-force characterisations and library routines.
"""
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "cu_8_16_24.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------- hand-worked tables
def check_handworked_dcs(o):
    g = golden()
    cu = np.array(g["cu_seqlens"], dtype=np.int32)
    for w_str, tab in g["dual_chunk_swap"].items():
        if not w_str.isdigit():
            continue
        W = int(w_str)
        for r in range(W):
            rows = o.rank_rows(cu, 48, W, o.DUAL_CHUNK_SWAP, r)
            assert rows.tolist() == tab["rows"][r], (W, r, rows.tolist())
        local, n_local = o.local_cu_seqlens(cu, 48, W, o.DUAL_CHUNK_SWAP)
        assert local.tolist() == tab["local_cu"], (W, local.tolist())
        assert n_local.tolist() == tab["n_local"]


def check_handworked_pc(o):
    g = golden()
    cu = np.array(g["cu_seqlens"], dtype=np.int32)
    for w_str, tab in g["packed_contiguous"].items():
        W = int(w_str)
        for r in range(W):
            rows = o.rank_rows(cu, 48, W, o.PACKED_CONTIGUOUS, r)
            assert rows.tolist() == tab["rows"][r]
        local, n_local = o.local_cu_seqlens(cu, 48, W, o.PACKED_CONTIGUOUS)
        assert local.tolist() == tab["local_cu"], (W, local.tolist())
        assert n_local.tolist() == tab["n_local"], (W, n_local.tolist())


def check_handworked_rejections(o):
    g = golden()
    cu = g["cu_seqlens"]
    for W in g["dual_chunk_swap"]["rejected_cp_sizes"]:
        assert "doc_not_divisible" in o.cu_violations(cu, 48, W, o.DUAL_CHUNK_SWAP)
    for W in (1, 2, 4):
        assert o.cu_violations(cu, 48, W, o.DUAL_CHUNK_SWAP) == set()
    assert "total_not_divisible" in o.cu_violations(cu, 48, 5, o.PACKED_CONTIGUOUS)
    assert o.cu_violations([1, 8, 48], 48, 1, o.PACKED_CONTIGUOUS) == {"first_not_zero"}
    assert o.cu_violations([0, 30, 24, 48], 48, 2, o.PACKED_CONTIGUOUS) == {"decreasing"}
    assert o.cu_violations([0, 8, 24, 40], 48, 2, o.PACKED_CONTIGUOUS) == {"last_not_total"}


def check_integer_grad_return(o):
    """G_w[t,h,d] = (w+1)(t+1) makes every sum exact: out = (t+1) W(W+1)/2."""
    g = golden()
    cu = np.array(g["cu_seqlens"], dtype=np.int32)
    T, H, D = 48, 2, 8
    t = np.arange(T, dtype=np.float32)[:, None, None]
    for W in (1, 2, 4):
        grads = [np.broadcast_to((w + 1) * (t + 1), (T, H, D)).astype(np.float32) for w in range(W)]
        for fn in ("grad_return", "grad_return_fused"):
            res = getattr(o, fn)(grads, cu, W, "f32", "f32")
            out = res[1] if fn == "grad_return" else res
            for owner in range(W):
                rows = np.array(g["dual_chunk_swap"][str(W)]["rows"][owner]) if str(W) in g["dual_chunk_swap"] \
                    else np.arange(T)
                want = (rows + 1) * (W * (W + 1) // 2)
                assert out[owner].shape == (T // W, H, D)
                assert (out[owner] == want[:, None, None].astype(np.float32)).all(), (fn, W, owner)
        if W == 2:
            out = o.grad_return(grads, cu, W, "f32", "f32")[1]
            assert out[0][:5, 0, 0].tolist() == g["integer_grad_return_w2"]["owner0_first"]
            assert out[1][:5, 0, 0].tolist() == g["integer_grad_return_w2"]["owner1_first"]
        # the same integers are exact in bf16
        gb = [o.f32_to_bf16_rne(x) for x in grads]
        out_b = o.grad_return_fused(gb, cu, W, "bf16", "bf16")
        for owner in range(W):
            rows = o.rank_rows(cu, T, W, o.DUAL_CHUNK_SWAP, owner)
            want = ((rows + 1) * (W * (W + 1) // 2)).astype(np.float32)
            assert (o.bf16_to_f32(out_b[owner][:, 0, 0]) == want).all()


# ---------------------------------------------------------------- order and seed
def check_sum_order(o):
    """(1e8 + 1) - 1e8 + 1 = 1 in fp32 only when slots are added 0,1,2,3 in turn."""
    vals = [1e8, 1.0, -1e8, 1.0]
    slots = [np.full((5,), v, dtype=np.float32) for v in vals]
    out = o.slot_sum(slots, "f32", "f32")
    assert (out == np.float32(1.0)).all(), out
    # a different order (3,2,1,0) would give 1 - 1e8 + 1 + 1e8 = 0, and (0,2,1,3) gives 2
    rev = o.slot_sum(slots[::-1], "f32", "f32")
    assert (rev == np.float32(0.0)).all(), rev
    # the same order through the fused path (writers hold constant rows)
    cu = np.array([0, 8], dtype=np.int32)
    grads = [np.full((8, 1, 1), v, dtype=np.float32) for v in vals]
    fused = o.grad_return_fused(grads, cu, 4, "f32", "f32")
    for owner in range(4):
        assert (fused[owner] == np.float32(1.0)).all()


def check_negative_zero_seed(o):
    """All slots -0.0 must give -0.0: the accumulator starts from slot 0, not +0."""
    for W in (1, 2, 4):
        slots = [np.full((3,), -0.0, dtype=np.float32) for _ in range(W)]
        out = o.slot_sum(slots, "f32", "f32")
        assert (out.view(np.uint32) == np.uint32(0x80000000)).all(), (W, out.view(np.uint32))
        out_b = o.slot_sum([o.f32_to_bf16_rne(s) for s in slots], "bf16", "bf16")
        assert (out_b == np.uint16(0x8000)).all()


# ---------------------------------------------------------------- bf16
def check_bf16_rne_against_torch(o, exhaustive=False):
    """fp32 -> bf16 must agree with torch's CPU cast (round-to-nearest-even)."""
    import torch

    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0x0000, 0x0001, 0x3FFF, 0x7FFF, 0x8000, 0x8001, 0xBFFF, 0xC000, 0xFFFF],
                    dtype=np.uint32)
    rng = np.random.default_rng(1234)
    lows = np.concatenate([lows, rng.integers(0, 1 << 16, size=7, dtype=np.uint32)])
    chunks = [(hi[:, None] | lows[None, :]).ravel()]
    chunks.append(rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32))
    if exhaustive:
        chunks = (np.arange(s, s + (1 << 26), dtype=np.uint64).astype(np.uint32)
                  for s in range(0, 1 << 32, 1 << 26))
    for bits in chunks:
        check_bf16_rne_bits(o, bits)


def check_bf16_rne_bits(o, bits):
    """The oracle's fp32 -> bf16 rounding of the fp32 values with bit patterns
    `bits` (uint32) against torch's CPU cast; a NaN must stay a quiet NaN with
    its sign (torch's NaN payload is not compared)."""
    import torch

    f = bits.view(np.float32)
    ours = o.f32_to_bf16_rne(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f)
    assert (ours[~nan] == ref[~nan]).all()
    # NaN: quiet, sign kept
    assert ((ours[nan] & 0x7FC0) == 0x7FC0).all()
    assert ((ours[nan] >> 15) == (bits[nan] >> 31)).all()


def check_bf16_widen_exact(o):
    u = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = o.bf16_to_f32(u)
    import torch

    ref = torch.from_numpy(u.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    same = (f.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(f) & np.isnan(ref))
    assert same.all()


# ---------------------------------------------------------------- special cases
def check_w1_identity(o, x=None):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((30, 3, 4)).astype(np.float32)
    for pol, cu in ((o.DUAL_CHUNK_SWAP, [0, 4, 10, 30]), (o.PACKED_CONTIGUOUS, [0, 7, 30])):
        parts = o.partition(x, np.array(cu), 1, pol)
        assert parts.shape == (1, 30, 3, 4)
        assert (parts[0] == x).all()


def check_single_document_native_layout(o):
    """One document: rank r holds [r c, (r+1) c) then [(2W-1-r) c, (2W-r) c), c = T/2W."""
    for W in (1, 2, 3, 4, 8):
        T = 2 * W * 5
        cu = np.array([0, T], dtype=np.int32)
        c = T // (2 * W)
        for r in range(W):
            want = list(range(r * c, (r + 1) * c)) + list(range((2 * W - 1 - r) * c, (2 * W - r) * c))
            assert o.rank_rows(cu, T, W, o.DUAL_CHUNK_SWAP, r).tolist() == want


def check_pc_is_reshape(o):
    rng = np.random.default_rng(6)
    for W in (1, 2, 4, 8):
        T = 8 * 9
        x = rng.standard_normal((T, 2, 3)).astype(np.float32)
        cu = np.array([0, 5, 5, 40, T], dtype=np.int32)
        parts = o.partition(x, cu, W, o.PACKED_CONTIGUOUS)
        assert (parts == x.reshape(W, T // W, 2, 3)).all()


# ---------------------------------------------------------------- brute force
def brute_owner_rows(cu, T, W):
    """Owner of every token by scanning documents and chunks; rows listed in global order.

    Token t in document b at offset j falls in chunk k = j // (L_b / 2W); chunk k
    belongs to rank k if k < W, else to rank 2W-1-k.  Under the stated local order
    (document-major, the lower chunk first, tokens ascending) a rank's local rows
    are its tokens in ascending global order.
    """
    owners = []
    for t in range(T):
        b = 0
        while not (cu[b] <= t < cu[b + 1]):
            b += 1
        L = cu[b + 1] - cu[b]
        c = L // (2 * W)
        k = (t - cu[b]) // c
        owners.append(k if k < W else 2 * W - 1 - k)
    return [[t for t in range(T) if owners[t] == r] for r in range(W)]


def check_brute_force_grad_return(o, seed=0):
    rng = np.random.default_rng(seed)
    for W, lengths in ((2, [4, 0, 8, 12]), (3, [6, 12]), (4, [8, 16, 8])):
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        T = int(cu[-1])
        H, D = 2, 3
        grads = [(rng.standard_normal((T, H, D)) * 10.0 ** int(rng.integers(-3, 3))).astype(np.float32)
                 for _ in range(W)]
        owner_rows = brute_owner_rows(cu, T, W)
        slots, out = o.grad_return(grads, cu, W, "f32", "f32")
        fused = o.grad_return_fused(grads, cu, W, "f32", "f32")
        for owner in range(W):
            assert o.rank_rows(cu, T, W, o.DUAL_CHUNK_SWAP, owner).tolist() == owner_rows[owner]
            for i, t in enumerate(owner_rows[owner]):
                for w in range(W):
                    assert (slots[owner][w][i] == grads[w][t]).all()
                for h in range(H):
                    for d in range(D):
                        acc = np.float32(grads[0][t, h, d])
                        for w in range(1, W):
                            acc = np.float32(acc + np.float32(grads[w][t, h, d]))
                        assert out[owner][i, h, d].view(np.uint32) == acc.view(np.uint32)
                        assert fused[owner][i, h, d].view(np.uint32) == acc.view(np.uint32)


# ---------------------------------------------------------------- invariants
def check_invariants(o, cu, T, W, policy, x):
    cu = np.asarray(cu, dtype=np.int32)
    B = len(cu) - 1
    n = T // W
    parts = o.partition(x, cu, W, policy)
    assert parts.shape == (W, n) + x.shape[1:]
    back = o.gather(parts, cu, W, policy)
    assert back.tobytes() == x.tobytes()
    all_rows = np.concatenate([o.rank_rows(cu, T, W, policy, r) for r in range(W)])
    assert sorted(all_rows.tolist()) == list(range(T))           # each token owned once
    for r in range(W):
        rows = o.rank_rows(cu, T, W, policy, r)
        assert (parts[r] == x[rows]).all()
        counts = np.array([((rows >= cu[b]) & (rows < cu[b + 1])).sum() for b in range(B)])
        if policy == o.DUAL_CHUNK_SWAP:
            assert (counts == (cu[1:] - cu[:-1]) // W).all()         # L_b / W per rank
    per_doc = np.zeros(B, dtype=np.int64)
    for r in range(W):
        rows = o.rank_rows(cu, T, W, policy, r)
        per_doc += np.array([((rows >= cu[b]) & (rows < cu[b + 1])).sum() for b in range(B)],
                            dtype=np.int64)
    assert (per_doc == cu[1:] - cu[:-1]).all()                       # document counts kept
    local, n_local = o.local_cu_seqlens(cu, T, W, policy)
    for r in range(W):
        lc = local[r]
        assert lc[0] == 0 and (np.diff(lc) >= 0).all() and lc[-1] == n
        k = n_local[r]
        assert lc[k] == n and (lc[k:] == n).all()
        if policy == o.DUAL_CHUNK_SWAP:
            assert (lc == cu // W).all()
        else:
            clipped = np.clip(cu.astype(np.int64) - r * n, 0, n)
            compact = np.unique(np.concatenate([[0], clipped, [n]]))
            assert lc[:k + 1].tolist() == compact.tolist()
            # the local segments are exactly the runs of each document inside the slice
            rows = o.rank_rows(cu, T, W, policy, r)
            doc_of = np.searchsorted(cu, rows, side="right") - 1
            starts = sorted({0, n} | {i for i in range(1, n) if doc_of[i] != doc_of[i - 1]})
            assert lc[:k + 1].tolist() == starts
    if policy == o.DUAL_CHUNK_SWAP and W > 0:
        # causal work per rank (keys seen by each query token) is balanced
        work = []
        for r in range(W):
            rows = o.rank_rows(cu, T, W, policy, r)
            doc_of = np.searchsorted(cu, rows, side="right") - 1
            work.append(int((rows - cu[doc_of] + 1).sum()))
        assert len(set(work)) == 1, work


def check_rank_row_matches_rank_rows(o):
    """The one-row form agrees with the full-array form, row by row."""
    rng = np.random.default_rng(9)
    for W in (1, 2, 3, 4, 8):
        for pol in o.POLICIES:
            if pol == o.DUAL_CHUNK_SWAP:
                lengths = [2 * W * int(k) for k in rng.integers(0, 4, size=6)]
            else:
                lengths = [int(k) for k in rng.integers(0, 9, size=6)]
                lengths[-1] += (-sum(lengths)) % W
            cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
            T = int(cu[-1])
            for r in range(W):
                rows = o.rank_rows(cu, T, W, pol, r)
                assert [o.rank_row(cu, T, W, pol, r, i) for i in range(len(rows))] == rows.tolist()


def check_fused_equals_unfused(o, seed=3):
    rng = np.random.default_rng(seed)
    for W, dt in ((2, "f32"), (4, "bf16"), (8, "bf16"), (3, "f32")):
        lengths = [2 * W * int(k) for k in rng.integers(0, 4, size=5)]
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        T = int(cu[-1])
        g32 = [rng.standard_normal((T, 2, 4)).astype(np.float32) for _ in range(W)]
        grads = g32 if dt == "f32" else [o.f32_to_bf16_rne(g) for g in g32]
        for out_dt in (("f32",) if dt == "f32" else ("bf16", "f32")):
            _, out = o.grad_return(grads, cu, W, dt, out_dt)
            fused = o.grad_return_fused(grads, cu, W, dt, out_dt)
            for owner in range(W):
                assert out[owner].tobytes() == fused[owner].tobytes()


# ---------------------------------------------------------------- accumulate mode, packed-contiguous owners
def check_accumulate_order(o):
    """Accumulating into 1e8 the slots (1, -1e8, 1) one at a time gives 1 in fp32.

    Adding the slot sum to the old value in one step would give 0 (1 - 1e8 + 1
    rounds to -1e8), and leaving the old value out would give -1e8.
    """
    slots = [np.full((5,), v, dtype=np.float32) for v in (1.0, -1e8, 1.0)]
    into = np.full((5,), 1e8, dtype=np.float32)
    assert (o.slot_sum(slots, "f32", "f32", into=into) == np.float32(1.0)).all()
    assert (into == np.float32(1e8)).all()  # the caller's array is not modified
    cu = np.array([0, 6], dtype=np.int32)
    grads = [np.full((6, 1, 1), v, dtype=np.float32) for v in (1.0, -1e8, 1.0)]
    for pol in (o.DUAL_CHUNK_SWAP, o.PACKED_CONTIGUOUS):
        into_o = [np.full((2, 1, 1), 1e8, dtype=np.float32) for _ in range(3)]
        fused = o.grad_return_fused(grads, cu, 3, "f32", "f32", policy=pol, into=into_o)
        _, out = o.grad_return(grads, cu, 3, "f32", "f32", policy=pol, into=into_o)
        for owner in range(3):
            assert (fused[owner] == np.float32(1.0)).all() and (out[owner] == np.float32(1.0)).all()


def check_accumulate_integer(o):
    """Old gradient 100(t+1) plus writers (w+1)(t+1): out = (t+1)(100 + W(W+1)/2), exact."""
    g = golden()
    cu = np.array(g["cu_seqlens"], dtype=np.int32)
    T, H, D = 48, 2, 4
    t = np.arange(T, dtype=np.float32)[:, None, None]
    for W in (1, 2, 4):
        grads = [np.broadcast_to((w + 1) * (t + 1), (T, H, D)).astype(np.float32) for w in range(W)]
        for pol in (o.DUAL_CHUNK_SWAP, o.PACKED_CONTIGUOUS):
            table = g[pol].get(str(W))
            rows = [np.array(table["rows"][r]) if table else np.arange(T) for r in range(W)]
            into = [np.broadcast_to(100 * (rows[r] + 1.0)[:, None, None], (T // W, H, D)).astype(np.float32)
                    for r in range(W)]
            want = [((rows[r] + 1) * (100 + W * (W + 1) // 2)).astype(np.float32)[:, None, None] for r in range(W)]
            _, out = o.grad_return(grads, cu, W, "f32", "f32", policy=pol, into=into)
            fused = o.grad_return_fused(grads, cu, W, "f32", "f32", policy=pol, into=into)
            # bf16 writers (the integers are exact in bf16) into an fp32 gradient
            gb = [o.f32_to_bf16_rne(x) for x in grads]
            fused_b = o.grad_return_fused(gb, cu, W, "bf16", "f32", policy=pol, into=into)
            for r in range(W):
                for res in (out, fused, fused_b):
                    assert (res[r] == want[r]).all(), (pol, W, r)
    # bf16 into bf16: T = 8, W = 2, sums stay below 256 (exact in bf16)
    cu8 = np.array([0, 8], dtype=np.int32)
    t8 = np.arange(8, dtype=np.float32)[:, None, None]
    grads = [o.f32_to_bf16_rne(np.broadcast_to((w + 1) * (t8 + 1), (8, 1, 2)).astype(np.float32)) for w in range(2)]
    for pol in (o.DUAL_CHUNK_SWAP, o.PACKED_CONTIGUOUS):
        rows = [o.rank_rows(cu8, 8, 2, pol, r) for r in range(2)]
        into = [o.f32_to_bf16_rne(np.broadcast_to(4.0 * (rows[r] + 1)[:, None, None], (4, 1, 2)).astype(np.float32))
                for r in range(2)]
        res = o.grad_return_fused(grads, cu8, 2, "bf16", "bf16", policy=pol, into=into)
        for r in range(2):
            assert (o.bf16_to_f32(res[r][:, 0, 0]) == 7.0 * (rows[r] + 1)).all()


def check_accumulate_signed_zero(o):
    """-0 into -0 slots stays -0; +0 into -0 slots gives +0 (IEEE: +0 + -0 = +0)."""
    for W in (1, 3):
        slots = [np.full((3,), -0.0, dtype=np.float32) for _ in range(W)]
        neg = o.slot_sum(slots, "f32", "f32", into=np.full((3,), -0.0, dtype=np.float32))
        pos = o.slot_sum(slots, "f32", "f32", into=np.zeros((3,), dtype=np.float32))
        assert (neg.view(np.uint32) == np.uint32(0x80000000)).all()
        assert (pos.view(np.uint32) == np.uint32(0)).all()


def check_pc_grad_return_is_reshape(o, seed=5):
    """Under packed-contiguous, owner o's slot from writer w is rows [o n, (o+1) n) of G_w."""
    rng = np.random.default_rng(seed)
    for W, lengths in ((2, [3, 0, 9]), (3, [5, 1, 6]), (4, [16])):
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        T = int(cu[-1])
        n = T // W
        grads = [rng.standard_normal((T, 2, 3)).astype(np.float32) for _ in range(W)]
        slots, out = o.grad_return(grads, cu, W, "f32", "f32", policy=o.PACKED_CONTIGUOUS)
        fused = o.grad_return_fused(grads, cu, W, "f32", "f32", policy=o.PACKED_CONTIGUOUS)
        for owner in range(W):
            for w in range(W):
                assert (slots[owner][w] == grads[w].reshape(W, n, 2, 3)[owner]).all()
            # per element, brute force: the writers' values at global token owner*n + i, in order
            for i in range(n):
                for h in range(2):
                    for d in range(3):
                        acc = np.float32(grads[0][owner * n + i, h, d])
                        for w in range(1, W):
                            acc = np.float32(acc + grads[w][owner * n + i, h, d])
                        assert out[owner][i, h, d].view(np.uint32) == acc.view(np.uint32)
                        assert fused[owner][i, h, d].view(np.uint32) == acc.view(np.uint32)


# ---------------------------------------------------------------- attention steps
def check_attention_handworked(o):
    g = golden()
    cu = np.array(g["cu_seqlens"], dtype=np.int32)
    for pol, table in (("dual_chunk_swap", g["attention_steps"]["dual_chunk_swap"]),
                       ("packed_contiguous", g["attention_steps"]["packed_contiguous"])):
        for W, ranks in table.items():
            for r, steps in enumerate(ranks):
                got = o.attention_steps(cu, 48, int(W), pol, r)
                assert [[list(seg) for seg in st] for st in got] == steps, (pol, W, r)


def brute_attention_pairs(cu, T):
    """Every (query token, key token) pair of causal document-isolated self-attention."""
    doc = np.zeros(T, dtype=np.int64)
    for b in range(len(cu) - 1):
        doc[int(cu[b]):int(cu[b + 1])] = b
    return {(t, s) for t in range(T) for s in range(t + 1) if doc[s] == doc[t]}


def check_attention_pairs(o, cu, T, W, pol):
    """The steps' pairs, with queries mapped to global tokens by the partition, are
    exactly the causal in-document pairs of the rank's tokens, each produced once,
    and every local row is a query of exactly one step."""
    want_all = brute_attention_pairs(cu, T)
    for r in range(W):
        rows = o.rank_rows(cu, T, W, pol, r)
        mine = set(rows.tolist())
        want = {(t, s) for (t, s) in want_all if t in mine}
        got, seen_rows = [], []
        for step in o.attention_steps(cu, T, W, pol, r):
            for q0, ql, k0, kl in step:
                assert 0 <= ql <= kl, (W, pol, r)
                for i in range(ql):
                    t = int(rows[q0 + i])
                    seen_rows.append(q0 + i)
                    got += [(t, s) for s in range(k0, k0 + kl - ql + i + 1)]
        assert sorted(seen_rows) == list(range(len(rows))), (W, pol, r)
        assert len(got) == len(set(got)) and set(got) == want, (W, pol, r)


def check_attention_brute_force(o):
    cases = [(2, "dual_chunk_swap", [4, 0, 8, 12]), (3, "dual_chunk_swap", [6, 12]),
             (2, "packed_contiguous", [3, 0, 9, 1, 7]), (3, "packed_contiguous", [5, 1, 6, 0, 3]),
             (4, "packed_contiguous", [16]), (4, "packed_contiguous", [1, 1, 1, 13]),
             (1, "dual_chunk_swap", [2, 4]), (1, "packed_contiguous", [3, 2])]
    for W, pol, lengths in cases:
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        check_attention_pairs(o, cu, int(cu[-1]), W, pol)


def check_attention_meta_closed_forms(o):
    """Packed per-step tables against closed forms: dual-chunk-swap cu_q = cu/(2W),
    cu_kv = (k+1) cu/(2W), q_offsets = cu/W (+ the chunk length in step 1),
    kv_offsets = cu; packed-contiguous cu_q = q_offsets = the local cu, cu_kv = the
    local cu shifted by the look-back to the first document's start."""
    cu = np.array([0, 12, 12, 36, 60, 96], dtype=np.int32)
    T, B = 96, 5
    for W in (1, 2, 3):
        m = o.attention_meta(cu, T, W, o.DUAL_CHUNK_SWAP)
        n = T // W
        for r in range(W):
            for s, k in ((0, r), (1, 2 * W - 1 - r)):
                assert (m["num_segments"][r, s] == B)
                assert (m["cu_seqlens_q"][r, s] == cu // (2 * W)).all()
                assert (m["cu_seqlens_kv"][r, s] == (k + 1) * (cu // (2 * W))).all()
                qo = cu[:-1] // W + s * (np.diff(cu) // (2 * W))
                assert (m["q_offsets"][r, s] == np.append(qo, n)).all()
                assert (m["kv_offsets"][r, s] == np.append(cu[:-1], T)).all()
                assert m["max_seqlen_q"][r, s] == np.diff(cu).max() // (2 * W)
                assert m["max_seqlen_kv"][r, s] == (k + 1) * (np.diff(cu).max() // (2 * W))
    cu = np.array([0, 5, 5, 17, 18, 30], dtype=np.int32)
    T = 30
    for W in (1, 2, 3, 5):
        n = T // W
        m = o.attention_meta(cu, T, W, o.PACKED_CONTIGUOUS)
        local, n_local = o.local_cu_seqlens(cu, T, W, o.PACKED_CONTIGUOUS)
        for r in range(W):
            d0 = int(np.searchsorted(cu, r * n, side="right")) - 1  # document of the first token
            back = r * n - int(cu[d0])
            assert m["num_segments"][r, 0] == n_local[r] and m["num_segments"][r, 1] == 0
            assert (m["cu_seqlens_q"][r, 0] == local[r]).all() and (m["q_offsets"][r, 0] == local[r]).all()
            kv = local[r] + back
            kv[0] = 0
            assert (m["cu_seqlens_kv"][r, 0] == kv).all()
            assert m["kv_offsets"][r, 0][0] == cu[d0]
            assert (m["cu_seqlens_q"][r, 1] == 0).all() and (m["q_offsets"][r, 1] == n).all()
            assert (m["kv_offsets"][r, 1] == T).all()


# ---------------------------------------------------------------- all-reduce (one-shot, ring)
def check_ring_chunks(o):
    # hand-worked: the plain equal split, q = ceil(n / W) elements per chunk,
    # W chunks covering [0, n), the last non-empty one shorter, empties at the end
    assert o.ring_chunks(300, 8) == [(0, 38), (38, 76), (76, 114), (114, 152), (152, 190),
                                     (190, 228), (228, 266), (266, 300)]
    assert o.ring_chunks(10, 4) == [(0, 3), (3, 6), (6, 9), (9, 10)]
    assert o.ring_chunks(9, 4) == [(0, 3), (3, 6), (6, 9), (9, 9)]
    assert o.ring_chunks(5, 8) == [(0, 1), (1, 2), (2, 3), (3, 4), (4, 5), (5, 5), (5, 5), (5, 5)]
    assert o.ring_chunks(1, 4) == [(0, 1), (1, 1), (1, 1), (1, 1)]
    assert o.ring_chunks(0, 3) == [(0, 0), (0, 0), (0, 0)]
    assert o.ring_chunks(4194304, 8)[1] == (524288, 1048576)   # 16 MiB of fp32, 8 ranks
    assert o.ring_chunks(100003, 7)[6] == (85722, 100003)      # q = 14287
    assert o.ring_chunks(1000, 1) == [(0, 1000)]
    for n in (0, 1, 63, 64, 65, 511, 512, 4097, 100000):
        for W in (1, 2, 3, 7, 8, 16):
            ch = o.ring_chunks(n, W)
            assert len(ch) == W and ch[0][0] == 0 and ch[-1][1] == n
            assert all(ch[k][1] == ch[k + 1][0] for k in range(W - 1))
            lens = [b - a for a, b in ch]
            full = [L for L in lens if L > 0]
            assert lens[:len(full)] == full           # empty chunks only at the end
            if len(full) <= 1:
                assert n <= 1 or W == 1
            else:
                # equal chunks but the last; their length is the smallest
                # with which W chunks cover n
                q = full[0]
                assert all(L == q for L in full[:-1]) and 0 < full[-1] <= q
                assert W * q >= n and W * (q - 1) < n


def check_allreduce_integer(o):
    # integer-valued fp32 data: every partial sum is exact, so both algorithms
    # give the exact integer sum on every rank, whatever the order
    rng = np.random.default_rng(11)
    for W in (1, 2, 3, 5, 8):
        for n in (0, 1, 64, 65, 300, 1030):
            ints = rng.integers(-1000, 1000, size=(W, n))
            xs = [r.astype(np.float32) for r in ints]
            exact = ints.sum(axis=0).astype(np.float64)
            for res in (o.allreduce_one_shot(xs, "f32"), o.allreduce_ring(xs, "f32"),
                        o.allreduce_two_shot(xs, "f32")):
                assert len(res) == W
                for r in range(W):
                    assert np.array_equal(res[r].astype(np.float64), exact), (W, n, r)


def _pattern(W, n, where):
    """Rank buffers of n fp32 elements where, inside chunk k, rank (k + j) % W
    holds where[j]."""
    xs = [np.zeros(n, dtype=np.float32) for _ in range(W)]
    q = n // W
    for k in range(W):
        for j, v in enumerate(where):
            xs[(k + j) % W][k * q:(k + 1) * q] = v
    return xs


def check_allreduce_order_handworked(o):
    # W = 4, n = 256: four chunks of 64.  2**24 + 1 is a tie in fp32 and rounds
    # to 2**24, while 2**24 + 2 is exact, so the order of adds shows in the result.
    big = np.float32(2 ** 24)
    # pattern A: inside chunk k, rank k holds 2^24, ranks k+2 and k+3 hold 1.
    # Ring order k, k+1, k+2, k+3 adds the ones after 2^24: 2^24 in every chunk.
    # Rank order 0..3 adds both ones first in chunks 2 and 3: 2^24 + 2 there.
    xs = _pattern(4, 256, [big, 0, 1, 1])
    ring = o.allreduce_ring(xs, "f32")
    one = o.allreduce_one_shot(xs, "f32")
    want_ring = [2 ** 24] * 4
    want_one = [2 ** 24, 2 ** 24, 2 ** 24 + 2, 2 ** 24 + 2]
    # pattern B: ranks k and k+1 hold 1, rank k+2 holds 2^24.  Ring order gives
    # 2 + 2^24 everywhere; a ring run the other way (k, k-1, ...) would give 2^24.
    xsb = _pattern(4, 256, [1, 1, big, 0])
    ringb = o.allreduce_ring(xsb, "f32")
    oneb = o.allreduce_one_shot(xsb, "f32")
    want_ringb = [2 ** 24 + 2] * 4
    want_oneb = [2 ** 24 + 2, 2 ** 24 + 2, 2 ** 24, 2 ** 24]
    # the two-shot sums every chunk in rank order, like the one-shot
    two = o.allreduce_two_shot(xs, "f32")
    twob = o.allreduce_two_shot(xsb, "f32")
    for r in range(4):
        for k in range(4):
            sl = slice(64 * k, 64 * (k + 1))
            assert (two[r][sl] == want_one[k]).all(), ("A two-shot", r, k)
            assert (twob[r][sl] == want_oneb[k]).all(), ("B two-shot", r, k)
            assert (ring[r][sl] == want_ring[k]).all(), ("A ring", r, k)
            assert (one[r][sl] == want_one[k]).all(), ("A one-shot", r, k)
            assert (ringb[r][sl] == want_ringb[k]).all(), ("B ring", r, k)
            assert (oneb[r][sl] == want_oneb[k]).all(), ("B one-shot", r, k)


def check_allreduce_bf16_rounding(o):
    # bf16 keeps 8 significant bits: 256 + 1 = 257 is a tie and rounds to 256
    # (0x4380); 258 is exact (0x4381).  Inside chunk k rank k holds 256 and the
    # others 1 (0x3F80).  The ring rounds after each add: 256 every time.  The
    # one-shot adds in fp32 and rounds once: 258.
    W, n = 3, 192
    xs = [np.full(n, 0x3F80, dtype=np.uint16) for _ in range(W)]
    for k in range(W):
        xs[k][64 * k:64 * (k + 1)] = 0x4380
    ring = o.allreduce_ring(xs, "bf16")
    one = o.allreduce_one_shot(xs, "bf16")
    two = o.allreduce_two_shot(xs, "bf16")
    for r in range(W):
        assert ring[r].dtype == np.uint16 and (ring[r] == 0x4380).all(), r
        assert one[r].dtype == np.uint16 and (one[r] == 0x4381).all(), r
        assert two[r].dtype == np.uint16 and (two[r] == 0x4381).all(), r


def check_allreduce_rotated_sums(o, seed=12):
    # closed form of the ring: chunk k is summed in rank order k, k+1, ..., k-1
    # (mod W), rounding to the buffer type after each add; every rank ends with
    # the same bits.  The one-shot and the two-shot equal the owner slot sum of
    # the W buffers.
    rng = np.random.default_rng(seed)
    for W, n in ((2, 130), (3, 1000), (5, 777), (8, 4096), (4, 3)):
        xs = [rng.standard_normal(n).astype(np.float32) for _ in range(W)]
        xb = [o.f32_to_bf16_rne(x) for x in xs]
        for data, dt in ((xs, "f32"), (xb, "bf16")):
            ring = o.allreduce_ring(data, dt)
            one = o.allreduce_one_shot(data, dt)
            want = np.empty_like(data[0])
            for k, (a, b) in enumerate(o.ring_chunks(n, W)):  # pinned by check_ring_chunks
                acc = data[k][a:b]
                for j in range(1, W):
                    x = data[(k + j) % W][a:b]
                    if dt == "f32":
                        acc = (acc + x).astype(np.float32)
                    else:
                        acc = o.f32_to_bf16_rne(o.bf16_to_f32(acc) + o.bf16_to_f32(x))
                want[a:b] = acc
            ref_one = o.slot_sum(data, dt, dt)
            two = o.allreduce_two_shot(data, dt)
            for r in range(W):
                assert np.array_equal(ring[r].view(np.uint8), want.view(np.uint8)), (W, n, dt, r)
                assert np.array_equal(one[r].view(np.uint8), ref_one.view(np.uint8)), (W, n, dt, r)
                assert np.array_equal(two[r].view(np.uint8), ref_one.view(np.uint8)), (W, n, dt, r)


def check_two_shot_chunk_owners(o):
    # every rank's chunk c must come from owner c's sum: give each rank's buffer a
    # different constant per chunk and check chunk c holds sum_w (1000 w + c)
    W, n = 5, 1000
    ch = o.ring_chunks(n, W)
    xs = [np.zeros(n, dtype=np.float32) for _ in range(W)]
    for w in range(W):
        for c, (a, b) in enumerate(ch):
            xs[w][a:b] = 1000 * w + c
    res = o.allreduce_two_shot(xs, "f32")
    for r in range(W):
        for c, (a, b) in enumerate(ch):
            assert (res[r][a:b] == 1000 * W * (W - 1) / 2 + W * c).all(), (r, c)


def check_allreduce_w1(o):
    x = np.random.default_rng(4).standard_normal(100).astype(np.float32)
    for res in (o.allreduce_ring([x], "f32"), o.allreduce_one_shot([x], "f32"),
                o.allreduce_two_shot([x], "f32")):
        assert len(res) == 1 and np.array_equal(res[0], x)


ALL_CHECKS = [
    check_handworked_dcs,
    check_handworked_pc,
    check_handworked_rejections,
    check_integer_grad_return,
    check_sum_order,
    check_negative_zero_seed,
    check_bf16_rne_against_torch,
    check_bf16_widen_exact,
    check_w1_identity,
    check_single_document_native_layout,
    check_pc_is_reshape,
    check_brute_force_grad_return,
    check_rank_row_matches_rank_rows,
    check_fused_equals_unfused,
    check_accumulate_order,
    check_accumulate_integer,
    check_accumulate_signed_zero,
    check_pc_grad_return_is_reshape,
    check_attention_handworked,
    check_attention_brute_force,
    check_attention_meta_closed_forms,
    check_ring_chunks,
    check_allreduce_integer,
    check_allreduce_order_handworked,
    check_allreduce_bf16_rounding,
    check_allreduce_rotated_sums,
    check_allreduce_w1,
    check_two_shot_chunk_owners,
]
