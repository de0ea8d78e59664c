"""CPU oracle for the THD context-parallel token layout and the owner gradient return.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only the
tests, the smoke check and the CPU-baseline leg of the benchmark call it.  It
shares no code, header, table or constant with the HIP library.

Everything here is a plain, slow, literal restatement of what the method
computes, in numpy (integer index arrays, fancy indexing as the gather
primitive, float32 adds one slot at a time).  Every function is exact: the
token layouts are permutations, and the gradient sums are defined by one fixed
order, so each output has exactly one correct bit pattern.

Sources (the pages; see their titles):
  * "[PyTorch] Add experimental packed-contiguous THD all-gather CP"
    (TransformerEngine PR 3221), sections "Conversation" (commit messages),
    "Why" and "Scope and constraints": the per-document DualChunkSwap partition
    (every document cut into 2*cp_size chunks) and the packed-contiguous policy
    (the whole physical buffer cut into cp_size equal chunks, document
    boundaries kept through per-rank sequence metadata).
  * "Add stream-ordered CP gradient return primitive" (TransformerEngine PR
    3235), sections "Description", "Sequence Diagram" and the author's reply
    on the ownership rule: owner o receives native sequence chunks o and
    2N-1-o; writers scatter global dK/dV into owner slots indexed
    [owner][writer], publish an epoch, owners wait for all epochs and then
    accumulate slots 0..cp_size-1.
  * "Low Latency Communication Kernels with NVSHMEM" (GPU MODE lecture 87
    notes), exercise list: the 1 KB - 16 MB sum sweep, and the all-reduce
    algorithms chosen by message size (one-shot against ring).

Readings where the pages are silent (the design notes list them all):
  * a DualChunkSwap rank stores its tokens document-major, and inside a
    document chunk r before chunk 2W-1-r, so its local cu_seqlens are cu/W;
  * a document whose length is not a multiple of 2W (DualChunkSwap) or a
    total length not a multiple of W (packed-contiguous) is rejected;
  * packed-contiguous local cu_seqlens are the sorted set of boundaries that
    fall inside the rank's slice, plus 0 and the slice length, padded with
    the slice length up to num_docs+1 entries;
  * by default the owner's output is overwritten with the sum; in the
    accumulate mode (the sequence diagram's "accumulate ... to dk" taken
    literally) the fp32 accumulator starts from the owner's current gradient
    and every slot is added to it in writer order;
  * otherwise the fp32 accumulator is seeded with slot 0 (so -0.0 survives)
    and slots are added in writer order 0..W-1;
  * the gradient return follows the metadata's policy: under packed-contiguous
    owner o's rows are its contiguous slice, as in the partition;
  * fp32 -> bf16 is round-to-nearest-even on the bit pattern; NaN stays a
    quiet NaN with its sign; denormals are kept;
  * attention after the all-gather is causal inside each document (token t
    sees token s when they share a document and s <= t), keys in global
    order; a dual-chunk-swap rank runs step 0 on chunk r and step 1 on chunk
    2W-1-r of every document, each against the document's prefix up to the
    chunk's end; a packed-contiguous rank runs one step in which every local
    segment sees its document from the first token on;
  * the all-reduce algorithms take their textbook forms: one-shot = every
    rank sums all W buffers in rank order, fp32, one rounding; ring = a
    reduce-scatter then an all-gather of W-1 steps each, passing to rank r+1,
    over W chunks of ceil(n/W) elements (the last ones shorter or empty); ring
    partials travel in the
    buffer type (a bf16 ring rounds after every add); the two-shot (not named by
    the pages; the direct two-step algorithm between the two) reduces chunk c at
    rank c in rank order, then every rank copies every reduced chunk.

bf16 tensors are represented here as numpy uint16 bit patterns.
"""
from __future__ import annotations

import numpy as np

DUAL_CHUNK_SWAP = "dual_chunk_swap"
PACKED_CONTIGUOUS = "packed_contiguous"
POLICIES = (DUAL_CHUNK_SWAP, PACKED_CONTIGUOUS)


# --------------------------------------------------------------------------
# cu_seqlens validation (PR 3221 "Scope and constraints"; PR 3235 reply on
# CP-size-generic ownership).
# --------------------------------------------------------------------------
def cu_violations(cu, total_tokens, cp_size, policy):
    """Return the set of named conditions a cu_seqlens array violates.

    Names: "first_not_zero", "decreasing", "last_not_total",
    "doc_not_divisible" (DualChunkSwap: some document length is not a multiple
    of 2*cp_size), "total_not_divisible" (packed-contiguous: total tokens not a
    multiple of cp_size).
    """
    cu = [int(v) for v in cu]
    bad = set()
    if cu[0] != 0:
        bad.add("first_not_zero")
    for b in range(len(cu) - 1):
        if cu[b + 1] < cu[b]:
            bad.add("decreasing")
    if cu[-1] != total_tokens:
        bad.add("last_not_total")
    if policy == DUAL_CHUNK_SWAP:
        for b in range(len(cu) - 1):
            if (cu[b + 1] - cu[b]) % (2 * cp_size) != 0:
                bad.add("doc_not_divisible")
    elif policy == PACKED_CONTIGUOUS:
        if total_tokens % cp_size != 0:
            bad.add("total_not_divisible")
    else:
        raise ValueError(policy)
    return bad


def _require_valid(cu, total_tokens, cp_size, policy):
    bad = cu_violations(cu, total_tokens, cp_size, policy)
    if bad:
        raise ValueError(f"invalid cu_seqlens for {policy}, W={cp_size}: {sorted(bad)}")


# --------------------------------------------------------------------------
# Ownership maps: which global token each rank's local rows hold.
# --------------------------------------------------------------------------
def dcs_rank_rows(cu, cp_size, rank):
    """Global token index of every local row of `rank` under DualChunkSwap.

    PR 3221 "Why": every sequence is divided into 2*cp_size chunks; PR 3235
    reply: owner o receives chunks o and 2N-1-o.  Each document is cut into
    2W equal chunks and the rank keeps chunk `rank` followed by chunk
    2W-1-rank, document after document.
    """
    W = cp_size
    pieces = []
    for b in range(len(cu) - 1):
        doc = np.arange(int(cu[b]), int(cu[b + 1]), dtype=np.int64)
        chunks = np.split(doc, 2 * W)  # raises unless len(doc) % 2W == 0
        pieces.append(chunks[rank])
        pieces.append(chunks[2 * W - 1 - rank])
    if not pieces:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate(pieces)


def pc_rank_rows(total_tokens, cp_size, rank):
    """Global token index of every local row of `rank` under packed-contiguous.

    PR 3221 commit messages: one contiguous chunk per CP rank, cp_size equal
    chunks; rank r holds tokens [r*T/W, (r+1)*T/W).
    """
    n = total_tokens // cp_size
    return np.arange(rank * n, (rank + 1) * n, dtype=np.int64)


def rank_rows(cu, total_tokens, cp_size, policy, rank):
    """Global token index of every local row of `rank` under `policy` (validated cu)."""
    _require_valid(cu, total_tokens, cp_size, policy)
    if policy == DUAL_CHUNK_SWAP:
        return dcs_rank_rows(cu, cp_size, rank)
    return pc_rank_rows(total_tokens, cp_size, rank)


def rank_row(cu, total_tokens, cp_size, policy, rank, i):
    """Global token of local row i of `rank`, one row at a time (for sampled checks).

    Walks the documents in order, counting the rows each one leaves on the rank
    (its two chunks under dual-chunk-swap), until the document holding local
    row i is reached; inside it, the first chunk-length rows come from chunk
    `rank` and the rest from chunk 2W-1-rank.  Packed-contiguous: r*T/W + i.
    Input validity is the caller's job (call cu_violations first).
    """
    W = cp_size
    if policy == PACKED_CONTIGUOUS:
        return rank * (total_tokens // W) + i
    seen = 0
    for b in range(len(cu) - 1):
        L = int(cu[b + 1]) - int(cu[b])
        c = L // (2 * W)
        if i < seen + 2 * c:
            j = i - seen
            chunk = rank if j < c else 2 * W - 1 - rank
            return int(cu[b]) + chunk * c + (j % c if c else 0)
        seen += 2 * c
    raise IndexError(i)


# --------------------------------------------------------------------------
# Per-rank sequence metadata (PR 3221: document boundaries retained through
# sequence metadata; packed metadata is one chunk per rank).
# --------------------------------------------------------------------------
def local_cu_seqlens(cu, total_tokens, cp_size, policy):
    """Per-rank local cu_seqlens, returned as (local_cu [W][B+1], n_local [W]).

    DualChunkSwap: each document contributes L_b/W tokens to every rank, so
    every rank's local cu is cu/W and holds all B documents.
    Packed-contiguous: rank r's slice [r*n, (r+1)*n) keeps every document
    boundary strictly inside it, shifted by -r*n, between 0 and n; the list
    is stored compact (n_local = its length - 1) and padded with n.
    """
    _require_valid(cu, total_tokens, cp_size, policy)
    W = cp_size
    B = len(cu) - 1
    local = np.zeros((W, B + 1), dtype=np.int32)
    n_local = np.zeros(W, dtype=np.int32)
    n = total_tokens // W
    for r in range(W):
        if policy == DUAL_CHUNK_SWAP:
            # Count the rows each document leaves on rank r (its two chunks).
            acc = 0
            local[r, 0] = 0
            for b in range(B):
                acc += len(dcs_rank_rows([cu[b], cu[b + 1]], W, r))
                local[r, b + 1] = acc
            n_local[r] = B
        else:
            lo, hi = r * n, (r + 1) * n
            bounds = {0, n}
            for v in cu:
                v = int(v)
                if lo < v < hi:
                    bounds.add(v - lo)
            ordered = sorted(bounds)
            n_local[r] = len(ordered) - 1
            row = ordered + [n] * (B + 1 - len(ordered))
            local[r, :] = row
    return local, n_local


# --------------------------------------------------------------------------
# Attention steps after the all-gather (PR 3221 "Why": the per-document
# partition runs two attention steps per rank, packed-contiguous one;
# "Scope and constraints": THD self-attention, all-gather CP, a full causal
# mask, no inter-sequence padding; document isolation kept by the metadata).
# --------------------------------------------------------------------------
def attention_steps(cu, total_tokens, cp_size, policy, rank):
    """Query and key ranges of every attention step of `rank`.

    Keys and values are the all-gathered buffer in global token order (the
    gather output).  Token t attends to token s when both lie in the same
    document and s <= t.  Returns a list of steps; a step is a list of segments
    (q_start, q_len, kv_start, kv_len): local query rows [q_start, q_start+q_len)
    whose keys are global rows [kv_start, kv_start+kv_len), the queries being
    the last q_len tokens of that key range (the causal mask aligned at the
    bottom right).

    DualChunkSwap: step 0 holds chunk `rank` of every document, step 1 chunk
    2W-1-rank; chunk k of a document with chunk length c attends to the
    document's first (k+1) c tokens.  Packed-contiguous: one step; every local
    segment (a document clipped to the rank's slice) attends from its
    document's first token up to its own last token.
    """
    _require_valid(cu, total_tokens, cp_size, policy)
    W = cp_size
    B = len(cu) - 1
    if policy == DUAL_CHUNK_SWAP:
        steps = []
        for step, chunk in ((0, rank), (1, 2 * W - 1 - rank)):
            segs = []
            first_local = 0  # local row of the document's first row on this rank
            for b in range(B):
                c = (int(cu[b + 1]) - int(cu[b])) // (2 * W)
                segs.append((first_local + step * c, c, int(cu[b]), (chunk + 1) * c))
                first_local += 2 * c
            steps.append(segs)
        return steps
    n = total_tokens // W
    local, n_local = local_cu_seqlens(cu, total_tokens, cp_size, policy)
    segs = []
    for j in range(int(n_local[rank])):
        q0, q1 = int(local[rank, j]), int(local[rank, j + 1])
        a = rank * n + q0  # global token of the segment's first query
        d = max(b for b in range(B) if int(cu[b]) <= a < int(cu[b + 1]))
        segs.append((q0, q1 - q0, int(cu[d]), a + (q1 - q0) - int(cu[d])))
    return [segs]


def attention_meta(cu, total_tokens, cp_size, policy):
    """The steps of every rank in the packed per-step form an attention call
    takes (two step records per rank; under packed-contiguous the second is
    empty).  For rank r, step s, with m segments:

      num_segments, max_seqlen_q, max_seqlen_kv, total_q, total_kv
      cu_seqlens_q[B+1]   0 then the running sum of q_len (padded with the total)
      cu_seqlens_kv[B+1]  the same for kv_len
      q_offsets[B+1]      q_start of each segment, then T/W (padded with T/W)
      kv_offsets[B+1]     kv_start of each segment, then T (padded with T)

    Returned as a dict of int32 arrays of shape [W, 2] (scalars) and
    [W, 2, B+1] (tables).
    """
    W = cp_size
    B = len(cu) - 1
    n = total_tokens // W
    out = {k: np.zeros((W, 2), dtype=np.int32)
           for k in ("num_segments", "max_seqlen_q", "max_seqlen_kv", "total_q", "total_kv")}
    for k in ("cu_seqlens_q", "cu_seqlens_kv", "q_offsets", "kv_offsets"):
        out[k] = np.zeros((W, 2, B + 1), dtype=np.int32)
    for r in range(W):
        steps = attention_steps(cu, total_tokens, cp_size, policy, r)
        for s in range(2):
            segs = steps[s] if s < len(steps) else []
            m = len(segs)
            q_len = [g[1] for g in segs]
            kv_len = [g[3] for g in segs]
            cq = [0] + [int(v) for v in np.cumsum(q_len)]
            ck = [0] + [int(v) for v in np.cumsum(kv_len)]
            out["num_segments"][r, s] = m
            out["max_seqlen_q"][r, s] = max(q_len, default=0)
            out["max_seqlen_kv"][r, s] = max(kv_len, default=0)
            out["total_q"][r, s] = cq[-1]
            out["total_kv"][r, s] = ck[-1]
            out["cu_seqlens_q"][r, s] = cq + [cq[-1]] * (B - m)
            out["cu_seqlens_kv"][r, s] = ck + [ck[-1]] * (B - m)
            out["q_offsets"][r, s] = [g[0] for g in segs] + [n] * (B + 1 - m)
            out["kv_offsets"][r, s] = [g[2] for g in segs] + [total_tokens] * (B + 1 - m)
    return out


# --------------------------------------------------------------------------
# Partition and inverse gather of a packed [T, H, D] tensor (bit copies).
# --------------------------------------------------------------------------
def partition(x, cu, cp_size, policy):
    """parts[r][i] = x[g_r(i)]; returns an array [W, T/W, ...] of x's dtype.

    "[PyTorch] Add experimental packed-contiguous THD all-gather CP", "Why":
    each rank's share of the packed buffer under the chosen policy.
    """
    T = x.shape[0]
    W = cp_size
    parts = np.empty((W, T // W) + x.shape[1:], dtype=x.dtype)
    for r in range(W):
        parts[r] = x[rank_rows(cu, T, W, policy, r)]
    return parts


def gather(parts, cu, cp_size, policy):
    """Inverse of partition: x[g_r(i)] = parts[r][i].

    Same page, commit messages: after the all-gather the dual-chunk-swap
    layout needs a reorder back to global order (packed-contiguous does not).
    """
    W = cp_size
    T = parts.shape[0] * parts.shape[1]
    x = np.empty((T,) + parts.shape[2:], dtype=parts.dtype)
    written = np.zeros(T, dtype=bool)
    for r in range(W):
        rows = rank_rows(cu, T, W, policy, r)
        assert not written[rows].any()
        x[rows] = parts[r]
        written[rows] = True
    assert written.all()
    return x


# --------------------------------------------------------------------------
# bf16 handling (bit patterns in uint16).
# --------------------------------------------------------------------------
def bf16_to_f32(u16):
    """Exact widening: the bf16 bits are the top half of the fp32 bits."""
    u16 = np.asarray(u16, dtype=np.uint16)
    return (u16.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(f32):
    """Round fp32 to bf16, nearest-even, on the bit pattern; NaN -> quiet NaN.

    The pages fix no rounding for the bf16 output; this is the stated reading
    (IEEE default rounding, as torch's cast): add 0x7FFF plus the lowest kept
    bit, keep the high 16 bits.
    """
    f32 = np.ascontiguousarray(f32, dtype=np.float32)
    u = f32.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint32)
    nan = np.isnan(f32)
    quiet = ((u >> np.uint64(16)) | np.uint64(0x0040)).astype(np.uint32)
    return np.where(nan, quiet, rounded).astype(np.uint16)


def _widen(a, dtype):
    if dtype == "f32":
        assert a.dtype == np.float32
        return a
    if dtype == "bf16":
        assert a.dtype == np.uint16
        return bf16_to_f32(a)
    raise ValueError(dtype)


def _narrow(acc, dtype):
    if dtype == "f32":
        return acc
    if dtype == "bf16":
        return f32_to_bf16_rne(acc)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# Owner gradient return (PR 3235 "Description" and "Sequence Diagram").
# --------------------------------------------------------------------------
def slot_sum(slots, in_dtype, out_dtype, into=None):
    """Sum W slot arrays in fp32, one add per slot, in writer order.

    Without `into` the accumulator is slot 0 and slots 1..W-1 are added.  With
    `into` (the owner's current gradient, in out_dtype) the accumulator starts
    from it and slots 0..W-1 are all added: "accumulate grad_key_return
    [0..cp_size-1] to dk" of the sequence diagram, one slot at a time.
    """
    if into is None:
        acc = _widen(slots[0], in_dtype).astype(np.float32, copy=True)
        rest = slots[1:]
    else:
        acc = _widen(into, out_dtype).astype(np.float32, copy=True)
        rest = slots
    with np.errstate(over="ignore", invalid="ignore"):  # IEEE: overflow -> inf, inf - inf -> NaN
        for s in rest:
            acc = (acc + _widen(s, in_dtype)).astype(np.float32)
    return _narrow(acc, out_dtype)


def _owner_list(cp_size, owners):
    return range(cp_size) if owners is None else [int(o) for o in owners]


def grad_scatter(grads, cu, cp_size, policy=DUAL_CHUNK_SWAP, owners=None):
    """Writer w puts the rows owner o owns into slot [o][w].

    grads: list over writers of global [T, ...] arrays.  Returns
    slots[o][w] = grads[w][g_o(:)], i.e. partition(grads[w])[o]: the two-chunk
    layout under DualChunkSwap, the owner's contiguous slice under
    packed-contiguous.  `owners` (default: all) restricts the work to those
    owners; the other owners' entries are None.  Every owner's slots depend on
    that owner's rows only, so a restricted call gives the same arrays.
    """
    W = cp_size
    T = grads[0].shape[0]
    slots = [[None] * W for _ in range(W)]
    for o in _owner_list(W, owners):
        rows = rank_rows(cu, T, W, policy, o)
        for w in range(W):
            slots[o][w] = grads[w][rows]
    return slots


def grad_return(grads, cu, cp_size, in_dtype, out_dtype, policy=DUAL_CHUNK_SWAP, into=None,
                owners=None):
    """Scatter, then each owner sums its W writer slots in order 0..W-1.

    Returns (slots, out) with out[o] = sum_w slots[o][w]; with `into` (a list
    over owners of their current gradients) out[o] = into[o] + slot 0 + ... .
    `owners` (default: all) restricts the work to those owners (None elsewhere).
    """
    slots = grad_scatter(grads, cu, cp_size, policy, owners)
    out = [None] * cp_size
    for o in _owner_list(cp_size, owners):
        out[o] = slot_sum(slots[o], in_dtype, out_dtype, None if into is None else into[o])
    return slots, out


def grad_return_fused(grads, cu, cp_size, in_dtype, out_dtype, policy=DUAL_CHUNK_SWAP, into=None,
                      owners=None):
    """No slots: out[o][i] = sum over w (in order) of grads[w][g_o(i)]
    (after into[o][i] when accumulating).  `owners` as in grad_return."""
    W = cp_size
    T = grads[0].shape[0]
    out = [None] * W
    for o in _owner_list(W, owners):
        rows = rank_rows(cu, T, W, policy, o)
        if into is None:
            acc = _widen(grads[0][rows], in_dtype).astype(np.float32, copy=True)
            first = 1
        else:
            acc = _widen(into[o], out_dtype).astype(np.float32, copy=True)
            first = 0
        with np.errstate(over="ignore", invalid="ignore"):
            for w in range(first, W):
                acc = (acc + _widen(grads[w][rows], in_dtype)).astype(np.float32)
        out[o] = _narrow(acc, out_dtype)
    return out


def epochs_after(cp_size, epoch):
    """Epoch table after every writer has published `epoch` to every owner.

    "Add stream-ordered CP gradient return primitive", "Sequence Diagram": each
    writer writes its epoch into every owner's [owner][writer] entry.
    """
    return np.full((cp_size, cp_size), epoch, dtype=np.uint32)


# --------------------------------------------------------------------------
# All-reduce of W rank buffers: one-shot and ring ("Low Latency Communication
# Kernels with NVSHMEM", the menu of all-reduce algorithms chosen by message
# size, and exercises 2-3: the 1 KB - 16 MB latency sweep, one-shot against
# ring).  The pages name the two algorithms without spelling them out; the
# textbook forms are taken:
#   * one-shot: every rank reads all W buffers and sums them itself, in rank
#     order 0..W-1, in fp32, rounding once to the buffer type;
#   * ring: the buffer is cut into W chunks; a reduce-scatter of W-1 steps in
#     which rank r passes one partial chunk to rank r+1 (mod W), which adds its
#     own contribution, then an all-gather of W-1 steps in which rank r passes
#     one complete chunk to rank r+1.  Partials travel in the buffer type, so a
#     bf16 ring rounds after every add.
# Buffers are one-dimensional arrays of n elements (f32, or bf16 as uint16).
# --------------------------------------------------------------------------
def ring_chunks(n, cp_size):
    """The buffer cut into W chunks for the ring: chunk k is
    [min(k*q, n), min((k+1)*q, n)) with q = ceil(n / W), the plain equal split.
    Every chunk but the last non-empty one holds q elements; trailing chunks are
    empty when (W-1)*q >= n (for instance n = 9, W = 4, or n < W)."""
    q = -(-n // cp_size)
    return [(min(k * q, n), min((k + 1) * q, n)) for k in range(cp_size)]


def allreduce_one_shot(inputs, dtype):
    """Every rank's result: sum of inputs[0..W-1] in rank order, fp32, one rounding."""
    W = len(inputs)
    acc = _widen(inputs[0], dtype).astype(np.float32, copy=True)
    with np.errstate(over="ignore", invalid="ignore"):
        for w in range(1, W):
            acc = (acc + _widen(inputs[w], dtype)).astype(np.float32)
    res = _narrow(acc, dtype)
    return [res.copy() for _ in range(W)]


def allreduce_ring(inputs, dtype):
    """The ring, simulated step by step with one working buffer per rank.

    Every step is a round of messages: each rank sends one chunk of its
    working buffer (as it stood before the step) to rank r+1, which stores
    it, after adding its own input chunk during the reduce-scatter.  In
    reduce-scatter step s rank r receives chunk (r-1-s) mod W; after W-1
    steps rank r holds chunk (r+1) mod W complete.  In all-gather step s
    rank r receives chunk (r-s) mod W, complete.
    """
    W = len(inputs)
    n = inputs[0].shape[0]
    chunks = ring_chunks(n, W)
    buf = [np.array(x, copy=True) for x in inputs]
    for s in range(W - 1):  # reduce-scatter
        msgs = []
        for r in range(W):
            src = (r - 1) % W
            a, b = chunks[(r - 1 - s) % W]
            msgs.append((r, a, b, buf[src][a:b].copy()))
        for r, a, b, m in msgs:
            with np.errstate(over="ignore", invalid="ignore"):
                acc = (_widen(m, dtype) + _widen(inputs[r][a:b], dtype)).astype(np.float32)
            buf[r][a:b] = _narrow(acc, dtype)
    for s in range(W - 1):  # all-gather
        msgs = []
        for r in range(W):
            a, b = chunks[(r - s) % W]
            msgs.append((r, a, b, buf[(r - 1) % W][a:b].copy()))
        for r, a, b, m in msgs:
            buf[r][a:b] = m
    return buf


def allreduce_two_shot(inputs, dtype):
    """Two-shot all-reduce: a reduce-scatter in which rank c sums chunk c of all W
    buffers itself (rank order, fp32, one rounding), then an all-gather in which every
    rank copies each other rank's reduced chunk.  Chunks as in the ring.

    The pages name one-shot and ring; this is the direct two-step algorithm that sits
    between them on a fully connected topology (each byte crosses a link twice, in two
    dependent steps), taken in its textbook form.
    """
    W = len(inputs)
    n = inputs[0].shape[0]
    chunks = ring_chunks(n, W)
    reduced = []
    for c in range(W):  # reduce-scatter: owner c pulls chunk c from every rank
        a, b = chunks[c]
        acc = _widen(inputs[0][a:b], dtype).astype(np.float32, copy=True)
        with np.errstate(over="ignore", invalid="ignore"):
            for w in range(1, W):
                acc = (acc + _widen(inputs[w][a:b], dtype)).astype(np.float32)
        reduced.append(_narrow(acc, dtype))
    out = [np.empty_like(inputs[0]) for _ in range(W)]
    for r in range(W):  # all-gather: rank r pulls every owner's chunk
        for c in range(W):
            a, b = chunks[c]
            out[r][a:b] = reduced[c]
    return out
