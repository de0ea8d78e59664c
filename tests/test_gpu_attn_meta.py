"""GPU parity of the attention-step metadata (cp_build_attn_meta) against the
CPU oracle: every field bit-exact for the hand-worked documents, random
documents (empty ones included) for W from 1 to 64 under both policies, more
documents than a workgroup has threads, the S=262144 layout workloads, empty
input, and the fail-closed paths (invalid metadata, a num_docs or cp_size that
differs from the metadata's)."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, O, WL, say

pytestmark = pytest.mark.gpu

POL = {0: O.DUAL_CHUNK_SWAP, 1: O.PACKED_CONTIGUOUS}


@pytest.fixture(scope="module")
def cp():
    from thd_token_layout_amd import cpthd
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return cpthd


def build_and_compare(cp, cu_np, T, W, policy):
    cu_np = np.asarray(cu_np, dtype=np.int32)
    meta = cp.cp_build_meta(torch.from_numpy(cu_np).to(DEV), T, W, policy, check=True)
    attn = cp.cp_build_attn_meta(meta)
    st = cp.cp_meta_status(meta)
    assert st[0] == cp.CP_OK, st
    magic, got = cp.read_attn_meta(attn, len(cu_np) - 1, W)
    assert magic == cp.CP_ATTN_MAGIC
    head = attn[:64].cpu().view(torch.int32)
    assert head[1:5].tolist() == [policy, W, len(cu_np) - 1, 2 if policy == 0 else 1]
    ref = O.attention_meta(cu_np, T, W, POL[policy])
    for k, v in ref.items():
        assert np.array_equal(got[k].numpy(), v), (k, W, policy)
    return meta, attn


@pytest.mark.parametrize("policy", [0, 1])
@pytest.mark.parametrize("W", [1, 2, 4])
def test_handworked_documents(cp, policy, W):
    say(f"case attention steps cu=[0,8,24,48] W={W} policy={policy}")
    build_and_compare(cp, [0, 8, 24, 48], 48, W, policy)


@pytest.mark.parametrize("policy", [0, 1])
@pytest.mark.parametrize("W,B", [(1, 5), (2, 9), (3, 17), (4, 40), (8, 7), (16, 3), (64, 12), (5, 300),
                                 (4, 3000)])
def test_random_documents(cp, policy, W, B):
    say(f"case attention steps random W={W} B={B} policy={policy}")
    rng = np.random.default_rng(W * 1000 + B + policy)
    if policy == 0:
        lengths = rng.integers(0, 5, size=B) * 2 * W
        lengths[rng.integers(0, B)] += 2 * W
    else:
        lengths = rng.integers(0, 30, size=B)
        lengths[rng.random(B) < 0.2] = 0
        lengths[-1] += (-int(lengths.sum())) % W + W
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    build_and_compare(cp, cu, int(cu[-1]), W, policy)


@pytest.mark.parametrize("name", ["dcs_s256k_w4", "pc_s256k_w4", "dcs1_s256k_w4", "dcs_t32k_w4", "pc_t64k_w4"])
def test_layout_workloads(cp, name):
    w = WL.WORKLOADS[name]
    say(f"case attention steps {name}")
    build_and_compare(cp, WL.cu_seqlens(w), w.total_tokens, w.cp_size, cp.POLICY[w.policy])


@pytest.mark.parametrize("policy", [0, 1])
def test_empty_input(cp, policy):
    say(f"case attention steps empty policy={policy}")
    build_and_compare(cp, [0], 0, 2, policy)
    build_and_compare(cp, [0, 0, 0, 0], 0, 4, policy)


def test_fail_closed(cp):
    say("case attention steps fail-closed")
    cu = torch.tensor([0, 8, 24, 48], dtype=torch.int32, device=DEV)
    # invalid cu_seqlens (a 9-token document under dual-chunk-swap W=2)
    bad = cp.cp_build_meta(torch.tensor([0, 9, 24, 48], dtype=torch.int32, device=DEV), 48, 2, 0)
    attn = torch.full((cp.cp_attn_meta_bytes(3, 2),), 0x5A, dtype=torch.uint8, device=DEV)
    cp.cp_build_attn_meta(bad, attn=attn)
    st, flags, _ = cp.cp_meta_status(bad)
    assert st == cp.CP_ERR_META and flags & cp.CP_CALL_USED_INVALID_META
    assert cp.read_attn_meta(attn, 3, 2)[0] == 0
    assert (attn[64:].cpu() == 0x5A).all()  # no record written
    # num_docs / cp_size that differ from the metadata's
    good = cp.cp_build_meta(cu, 48, 2, 0, check=True)
    attn = torch.full((cp.cp_attn_meta_bytes(4, 2),), 0x5A, dtype=torch.uint8, device=DEV)
    st = cp.lib.cp_build_attn_meta(good.ptr(), 4, 2, attn.data_ptr(), attn.numel(), None)
    assert st == cp.CP_OK
    st, flags, _ = cp.cp_meta_status(good)
    assert st == cp.CP_ERR_META and flags & cp.CP_CALL_DOCS_MISMATCH
    assert (attn[64:].cpu() == 0x5A).all()
    good = cp.cp_build_meta(cu, 48, 2, 0, check=True)
    attn = torch.full((cp.cp_attn_meta_bytes(3, 1),), 0x5A, dtype=torch.uint8, device=DEV)
    st = cp.lib.cp_build_attn_meta(good.ptr(), 3, 1, attn.data_ptr(), attn.numel(), None)
    assert st == cp.CP_OK
    st, flags, _ = cp.cp_meta_status(good)
    assert st == cp.CP_ERR_META and flags & cp.CP_CALL_CP_SIZE_MISMATCH
    assert (attn[64:].cpu() == 0x5A).all()
    # host-side: the output buffer overlaps the metadata
    buf = torch.empty(4096, dtype=torch.uint8, device=DEV)
    good = cp.cp_build_meta(cu, 48, 2, 0, meta=buf[:256], check=True)
    with pytest.raises(cp.CpError) as e:
        cp.cp_build_attn_meta(good, attn=buf[128:])
    assert e.value.status == cp.CP_ERR_ALIAS


def _attention(q, k, v, mask):
    """Plain fp32 softmax attention: q [Tq,H,D], k/v [Tk,H,D], mask [Tq,Tk] (True = attend)."""
    qh = q.permute(1, 0, 2).contiguous()
    kh = k.permute(1, 2, 0).contiguous()
    vh = v.permute(1, 0, 2).contiguous()
    s = torch.matmul(qh, kh) / float(q.shape[-1]) ** 0.5
    s = s.masked_fill(~mask[None], float("-inf"))
    return torch.matmul(torch.softmax(s, dim=-1), vh).permute(1, 0, 2)


@pytest.mark.parametrize("policy,lengths,W", [
    (0, [16, 48, 32, 64], 2), (0, [64, 16, 0, 48], 4),
    (1, [5, 40, 3, 0, 70, 10], 4), (1, [100, 7, 21], 2), (1, [128], 4)])
def test_tables_drive_document_causal_attention(cp, policy, lengths, W):
    """Attention run per rank and per step from the GPU-built tables (queries: the
    rank's local rows of each segment; keys/values: the gathered global buffer;
    causal mask aligned at the bottom right of each segment) and gathered back
    equals attention over the whole packed buffer with the causal in-document mask."""
    say(f"case attention through the tables, policy={policy} W={W}")
    cu_np = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T, B, H, D = int(cu_np[-1]), len(lengths), 2, 16
    meta = cp.cp_build_meta(torch.from_numpy(cu_np).to(DEV), T, W, policy, check=True)
    magic, tab = cp.read_attn_meta(cp.cp_build_attn_meta(meta), B, W)
    assert magic == cp.CP_ATTN_MAGIC
    gen = torch.Generator(device=DEV).manual_seed(T + W)
    q, k, v = (torch.randn((T, H, D), generator=gen, device=DEV) for _ in range(3))
    doc = torch.repeat_interleave(torch.arange(B, device=DEV), torch.tensor(lengths, device=DEV))
    pos = torch.arange(T, device=DEV)
    full_mask = (doc[:, None] == doc[None, :]) & (pos[None, :] <= pos[:, None])
    want = _attention(q, k, v, full_mask)
    q_local = cp.cp_partition_thd(q, meta)  # [W, T/W, H, D]
    out_local = torch.full_like(q_local, float("nan"))
    for r in range(W):
        for step in range(2):
            m = int(tab["num_segments"][r, step])
            cq, qo = tab["cu_seqlens_q"][r, step], tab["q_offsets"][r, step]
            ck, ko = tab["cu_seqlens_kv"][r, step], tab["kv_offsets"][r, step]
            for j in range(m):
                ql, kl = int(cq[j + 1] - cq[j]), int(ck[j + 1] - ck[j])
                q0, k0 = int(qo[j]), int(ko[j])
                if ql == 0:
                    continue
                i = torch.arange(ql, device=DEV)[:, None]
                kk = torch.arange(kl, device=DEV)[None, :]
                mask = kk <= (kl - ql) + i
                out_local[r, q0:q0 + ql] = _attention(q_local[r, q0:q0 + ql], k[k0:k0 + kl], v[k0:k0 + kl], mask)
    got = cp.cp_gather_thd(out_local, meta)
    assert not torch.isnan(got).any()
    assert torch.allclose(got, want, atol=1e-5, rtol=1e-5), (got - want).abs().max().item()
