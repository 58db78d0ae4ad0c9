"""GPU checks of the whole chain and of two invariants the pages state.

1. The exact tiny causal prefill (L = 1024, every position a query, H^I = 4,
   d^I = 64, k = 64, H = 8, d_c = 128, d_R = 32, fp32) run as one GPU chain:
   GPU indexer -> GPU top-k -> GPU sparse MLA over all 1024 rows.  The scores
   are exact multiples of 1/4, so the index sets must equal the oracle's bit
   for bit; the attention must be within 2e-3 of the oracle's on those sets
   ("Sparse Attention 数学学习笔记" §9 with the stated sizes).
2. Causality ("MLA 与稀疏注意力", the check that needs no training): in a
   causal prefill, changing the cache at positions after t must not change
   the selected set or the output of any query at a position <= t.  Checked
   bit for bit on the default prefill call and on the three-call path.
3. Placement ("Sparse Attention 数学学习笔记" §11, HiSparse: where the rows
   live does not change the attention): the same rows stored at permuted
   positions, with the index lists remapped slot for slot, or stored as a
   split cache instead of a packed one, give the same output bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import ATTN_ATOL_BF16, assert_attention_close, assert_index_sets
from top_indexer_sparse_amd import api, workloads

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def test_tiny_prefill_whole_chain_on_gpu():
    _announce("tiny prefill chain: GPU indexer -> GPU top-k -> GPU MLA, L=1024")
    wl = workloads.tiny_prefill()
    t = wl.to(DEV)
    s = api.sparse_attn_indexer_scores(t.q_idx, t.w, t.k_idx, q_pos=t.q_pos)
    idx, cnt = api.sparse_attn_topk(s, wl.topk, q_pos=t.q_pos)
    out, lse = api.sparse_attn_mla_forward(t.q_lat, t.q_rope, t.kv[..., :wl.dc],
                                           t.kv[..., wl.dc:], idx, wl.sm_scale)
    torch.cuda.synchronize()
    rs = oracle.indexer(wl.q_idx, wl.w, wl.k_idx, q_pos=wl.q_pos)
    oi, oc = oracle.topk(rs, wl.topk, q_pos=wl.q_pos)
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    assert np.array_equal(gc, oc), "counts differ from the oracle"
    assert np.array_equal(gi, oi), "index sets differ from the oracle (exact workload)"
    # rows t < 63 have t + 1 < k candidates: all of them, then -1 padding
    assert np.array_equal(gc[0, :64], np.arange(1, 65))
    ro, rl = oracle.sparse_mla(wl.q_lat, wl.q_rope, wl.kv, oi, wl.sm_scale, dc=wl.dc)
    err = assert_attention_close(out, ro, 2e-3, lse, rl)
    assert err < 1e-4  # fp32 arithmetic throughout


def _perturb_future(wl, t0, seed):
    """A copy of the prefill workload whose cache rows after position t0
    (indexer keys and latent rows) are replaced by fresh random values."""
    g = torch.Generator().manual_seed(seed)
    k_idx = wl.k_idx.clone()
    kv = wl.kv.clone()
    n = wl.L - t0 - 1
    k_idx[:, t0 + 1:] = (3.0 * torch.randn(wl.B, n, wl.dI, generator=g)).to(k_idx.dtype)
    kv[:, t0 + 1:] = (3.0 * torch.randn(wl.B, n, kv.shape[-1], generator=g)).to(kv.dtype)
    return k_idx, kv


@pytest.mark.parametrize("path", ["prefill_call", "three_calls"])
def test_causal_prefill_ignores_the_future(path):
    _announce(f"future perturbation, causal prefill L=700 ({path})")
    wl = workloads.prefill_16k(L=700, H=64, topk=128, n_needles=0)
    t0 = 333

    def run(k_idx, kv):
        t = wl.to(DEV)
        k_idx, kv = k_idx.to(DEV), kv.to(DEV)
        c, r = kv[..., :wl.dc], kv[..., wl.dc:]
        if path == "prefill_call":
            idx = torch.empty((wl.B, wl.T, wl.topk), dtype=torch.int32, device=DEV)
            out, lse = api.sparse_attn_prefill(t.q_idx, t.w, k_idx, wl.topk, t.q_lat, t.q_rope,
                                               c, r, wl.sm_scale, q_pos=t.q_pos, idx_out=idx)
        else:
            s = api.sparse_attn_indexer_scores(t.q_idx, t.w, k_idx, q_pos=t.q_pos)
            idx, _ = api.sparse_attn_topk(s, wl.topk, q_pos=t.q_pos)
            out, lse = api.sparse_attn_mla_forward(t.q_lat, t.q_rope, c, r, idx, wl.sm_scale)
        torch.cuda.synchronize()
        return idx.cpu(), out.cpu(), lse.cpu()

    i0, o0, l0 = run(wl.k_idx, wl.kv)
    k2, kv2 = _perturb_future(wl, t0, 99)
    i1, o1, l1 = run(k2, kv2)
    # queries at positions <= t0 see nothing of the change
    assert torch.equal(i0[:, :t0 + 1], i1[:, :t0 + 1])
    assert torch.equal(o0[:, :t0 + 1], o1[:, :t0 + 1])
    assert torch.equal(l0[:, :t0 + 1], l1[:, :t0 + 1])
    # and the change is visible after t0 (the perturbation is not a no-op)
    assert not torch.equal(o0[:, t0 + 1:], o1[:, t0 + 1:])
    # no selected position lies after its query
    gi = i0.numpy()[0]
    for q in range(wl.T):
        sel = gi[q][gi[q] >= 0]
        assert sel.size and sel.max() <= q


def test_placement_of_rows_does_not_change_the_output():
    _announce("placement: permuted rows, remapped slots; split vs packed cache")
    B, L, k, H = 3, 2600, 2048, 128
    wl = workloads.decode_32k(B=B, L=L, H=H, n_needles=16)
    rng = np.random.default_rng(7)
    idx = np.stack([np.sort(rng.choice(L, k, replace=False)) for _ in range(B)])[:, None]
    idx = idx.astype(np.int32)
    idx[0, 0, -5:] = -1
    perm = np.stack([rng.permutation(L) for _ in range(B)])       # new row p holds old perm[p]
    inv = np.argsort(perm, axis=1)                                 # old row s is at inv[s]
    kv_p = torch.stack([wl.kv[b][torch.from_numpy(perm[b])] for b in range(B)])
    idx_p = idx.copy()
    for b in range(B):
        ok = idx[b, 0] >= 0
        idx_p[b, 0, ok] = inv[b][idx[b, 0, ok]]
    ql, qr = wl.q_lat.to(DEV), wl.q_rope.to(DEV)
    kv, kvp = wl.kv.to(DEV), kv_p.to(DEV)
    g_idx, g_idxp = torch.from_numpy(idx).to(DEV), torch.from_numpy(idx_p).to(DEV)
    o0, l0 = api.sparse_attn_mla_forward(ql, qr, kv[..., :wl.dc], kv[..., wl.dc:], g_idx,
                                         wl.sm_scale)
    o1, l1 = api.sparse_attn_mla_forward(ql, qr, kvp[..., :wl.dc], kvp[..., wl.dc:], g_idxp,
                                         wl.sm_scale)
    # the same rows in a split cache: two tensors with their own row strides
    c_split = kv[..., :wl.dc].contiguous()
    r_split = kv[..., wl.dc:].contiguous()
    o2, l2 = api.sparse_attn_mla_forward(ql, qr, c_split, r_split, g_idx, wl.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1), "permuted placement changed the output"
    assert torch.equal(o0, o2) and torch.equal(l0, l2), "split cache changed the output"
    ro, rl = oracle.sparse_mla(wl.q_lat, wl.q_rope, wl.kv, idx, wl.sm_scale, dc=wl.dc)
    assert_attention_close(o0, ro, ATTN_ATOL_BF16, l0, rl)


def test_placement_fused_decode_selects_the_mapped_set():
    # the fused decode over a permuted cache (indexer keys and latent rows
    # moved together) selects the image of the same set; scores are continuous,
    # so the set rule (near-ties only) applies to both runs against the oracle
    _announce("placement: fused decode over a permuted cache")
    B, L = 2, 4500
    wl = workloads.decode_32k(B=B, L=L, n_needles=16)
    rng = np.random.default_rng(8)
    perm = np.stack([rng.permutation(L) for _ in range(B)])
    kidx_p = torch.stack([wl.k_idx[b][torch.from_numpy(perm[b])] for b in range(B)])
    kv_p = torch.stack([wl.kv[b][torch.from_numpy(perm[b])] for b in range(B)])

    def run(k_idx, kv):
        t = wl.to(DEV)
        k_idx, kv = k_idx.to(DEV), kv.to(DEV)
        out, lse, idx = api.sparse_attn_decode(t.q_idx, t.w, k_idx, None, None, wl.topk,
                                               t.q_lat, t.q_rope, kv[..., :wl.dc],
                                               kv[..., wl.dc:], wl.sm_scale)
        torch.cuda.synchronize()
        return out.cpu(), lse.cpu(), idx.cpu().numpy()

    o0, l0, i0 = run(wl.k_idx, wl.kv)
    o1, l1, i1 = run(kidx_p, kv_p)
    rs = oracle.indexer(wl.q_idx, wl.w, wl.k_idx)
    oi, oc = oracle.topk(rs, wl.topk)
    assert_index_sets(i0, (i0 >= 0).sum(-1), oi, oc, rs)
    # slot j of the permuted run holds new row i1[j], which is old row perm[i1[j]]
    mapped = np.full(i1.shape, -1, dtype=np.int64)
    for b in range(B):
        sel = i1[b, 0][i1[b, 0] >= 0]
        old = np.sort(perm[b][sel])
        mapped[b, 0, :old.size] = old
    assert_index_sets(mapped, (mapped >= 0).sum(-1), oi, oc, rs)
    # outputs on the two placements agree to the attention tolerance (the
    # slot order differs, so fp32 sums may round differently)
    assert float((o0 - o1).abs().max()) <= ATTN_ATOL_BF16
