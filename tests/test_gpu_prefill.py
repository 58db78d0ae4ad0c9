"""GPU parity of the prefill entry points.

sparse_attn_prefill_select (indexer scores and Top-K fused, the score row kept
on chip) must return exactly the index sets that the Top-K rule gives on the
same scores: the oracle's top-k applied to the scores of
sparse_attn_indexer_scores (which carry the same bits), bit for bit, plus the
set rule against the oracle's own fp64 scores.  sparse_attn_prefill is checked
in its three modes: sparse (the select, then the sparse MLA), dense (every
causal candidate, against the oracle's masked form) and auto.
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


def _select_both(t, k):
    """(fused idx, fused count, staged idx, staged count, GPU scores) on device tensors."""
    fi, fc = api.sparse_attn_prefill_select(t.q_idx, t.w, t.k_idx, k, k_scale=t.k_scale,
                                            q_pos=t.q_pos, kv_len=t.kv_len)
    s = api.sparse_attn_indexer_scores(t.q_idx, t.w, t.k_idx, k_scale=t.k_scale, q_pos=t.q_pos,
                                       kv_len=t.kv_len)
    si, sc = api.sparse_attn_topk(s, k, q_pos=t.q_pos, kv_len=t.kv_len)
    torch.cuda.synchronize()
    return fi.cpu().numpy(), fc.cpu().numpy(), si.cpu().numpy(), sc.cpu().numpy(), s


def _rule_topk(scores, k, q_pos, kv_len):
    """The selection rule by brute force (sort by (-score, position)), with the
    library's documented reading for non-finite scores: NaN and -inf are never
    candidates, +inf is the largest score.  For rows the strict oracle refuses."""
    B, T, L = scores.shape
    idx = np.full((B, T, k), -1, dtype=np.int64)
    cnt = np.zeros((B, T), dtype=np.int64)
    for b in range(B):
        for t_ in range(T):
            lim = L if kv_len is None else min(L, max(int(kv_len[b]), 0))
            if q_pos is not None:
                lim = min(lim, max(int(q_pos[b, t_]) + 1, 0))
            row = scores[b, t_, :lim]
            ok = ~np.isnan(row) & (row != -np.inf)
            pos = np.nonzero(ok)[0]
            order = np.lexsort((pos, -row[pos]))[:k]
            sel = np.sort(pos[order])
            idx[b, t_, :len(sel)] = sel
            cnt[b, t_] = len(sel)
    return idx, cnt


def _check_select(wl, fp64_rule=True, strict=True):
    t = wl.to(DEV)
    fi, fc, si, sc, s = _select_both(t, wl.topk)
    # the Top-K rule on the GPU's own scores: identical sets, bit for bit
    if strict:
        oi, oc = oracle.topk(s.cpu().double().numpy(), wl.topk, q_pos=wl.q_pos,
                             kv_len=wl.kv_len)
    else:
        oi, oc = _rule_topk(s.cpu().numpy(), wl.topk, wl.q_pos, wl.kv_len)
    assert np.array_equal(fc, oc), "counts differ from the oracle's top-k of the same scores"
    assert np.array_equal(fi, oi), "sets differ from the oracle's top-k of the same scores"
    assert np.array_equal(fc, sc) and np.array_equal(fi, si), "fused and staged paths differ"
    if fp64_rule:
        rs = oracle.indexer(wl.q_idx, wl.w, wl.k_idx, k_scale=wl.k_scale, q_pos=wl.q_pos,
                            kv_len=wl.kv_len)
        ri, rc = oracle.topk(rs, wl.topk, q_pos=wl.q_pos, kv_len=wl.kv_len)
        assert_index_sets(fi, fc, ri, rc, rs)
    return fi, fc


@pytest.mark.parametrize("case", [
    dict(B=2, T=3000, L=3000, HI=64, dI=128, topk=256),
    dict(B=2, T=1200, L=5000, HI=64, dI=128, topk=2048, fp8=True),
    dict(B=3, T=501, L=9000, HI=16, dI=64, topk=512, q_pos="spread", kv_len=[9000, 6000, 100]),
    dict(B=1, T=300, L=20000, HI=128, dI=128, topk=1024),
    dict(B=1, T=64, L=32768, HI=64, dI=128, topk=2048),
    dict(B=2, T=101, L=101, HI=32, dI=128, topk=300, fp8=True),
    dict(B=2, T=40, L=4000, HI=64, dI=64, topk=1, q_pos="spread"),
], ids=["causal3000", "fp8_k2048", "spread_ragged", "hi128_L20000", "maxL", "k_above_all",
        "k1"])
def test_prefill_select_matches_topk_of_the_scores(case):
    _announce(f"prefill_select {case}")
    wl = workloads.prefill_batch(with_mla=False, **case)
    _check_select(wl)


def _crafted(kind):
    """Index inputs that stress the select: ties, equal rows, narrow ranges,
    signed scores, NaN queries."""
    B, T, L, HI, dI, k = 2, 64, 6000, 16, 64, 700
    wl = workloads.prefill_batch(B=B, T=T, L=L, HI=HI, dI=dI, topk=k, with_mla=False)
    g = torch.Generator().manual_seed(77)
    if kind == "ties":
        # small integers: integer dot products, w in {1/4, 1/2}: many equal scores
        wl.q_idx = torch.randint(-2, 3, (B, T, HI, dI), generator=g).to(torch.bfloat16)
        wl.k_idx = torch.randint(-2, 3, (B, L, dI), generator=g).to(torch.bfloat16)
        wl.w = torch.randint(1, 3, (B, T, HI), generator=g).float() * 0.25
    elif kind == "allzero":
        wl.w = torch.zeros(B, T, HI)  # every score is +0.0: the lowest positions win
    elif kind == "narrow":
        # keys that differ in their last bits only: scores share their high bits
        base = torch.randn(1, 1, dI, generator=g)
        wl.k_idx = (base + 2.0 ** -7 * torch.randint(0, 4, (B, L, dI), generator=g)).to(torch.bfloat16)
    elif kind == "signed":
        wl.w = torch.rand(B, T, HI, generator=g) * 2 - 1  # negative head weights
    elif kind == "nan":
        # a NaN head weight makes every score of its row NaN: no candidate; an
        # infinite one gives +inf where that head's product is positive and
        # NaN (inf * 0) where its ReLU is zero
        wl.w[0, 5, 0] = float("nan")
        wl.w[1, 9, 3] = float("inf")
    return wl


@pytest.mark.parametrize("kind", ["ties", "allzero", "narrow", "signed", "nan"])
def test_prefill_select_crafted_scores(kind):
    _announce(f"prefill_select crafted {kind}")
    wl = _crafted(kind)
    fi, fc = _check_select(wl, fp64_rule=kind not in ("nan", "narrow"), strict=kind != "nan")
    if kind == "allzero":
        lim = wl.q_pos.numpy() + 1
        for b in range(wl.B):
            for t_ in range(wl.T):
                c = min(wl.topk, lim[b, t_])
                assert fc[b, t_] == c
                assert np.array_equal(fi[b, t_, :c], np.arange(c))
    if kind == "nan":
        assert fc[0, 5] == 0 and np.all(fi[0, 5] == -1)


def test_prefill_select_empty_rows():
    _announce("prefill_select empty rows")
    wl = workloads.prefill_batch(B=2, T=50, L=500, HI=64, dI=128, topk=64, with_mla=False,
                                 kv_len=[500, 0])
    wl.q_pos[0, :7] = -1
    fi, fc = _check_select(wl)
    assert np.all(fc[1] == 0) and np.all(fi[1] == -1)
    assert np.all(fc[0, :7] == 0)


# --------------------------------------------------------------------------
# sparse_attn_prefill: sparse, dense and auto modes
# --------------------------------------------------------------------------

def _prefill(t, wl, mode, idx_out=None):
    c_kv, k_rope = t.kv[..., :wl.dc], t.kv[..., wl.dc:]
    out, lse = api.sparse_attn_prefill(t.q_idx, t.w, t.k_idx, wl.topk, t.q_lat, t.q_rope, c_kv,
                                       k_rope, wl.sm_scale, k_scale=t.k_scale, q_pos=t.q_pos,
                                       kv_len=t.kv_len, mode=mode, idx_out=idx_out)
    torch.cuda.synchronize()
    return out, lse


def test_prefill_sparse_mode():
    _announce("prefill sparse B=2 T=L=600 H=64 k=128")
    wl = workloads.prefill_batch(B=2, T=600, L=600, HI=64, dI=128, topk=128, H=64)
    t = wl.to(DEV)
    idx = torch.empty((wl.B, wl.T, wl.topk), dtype=torch.int32, device=DEV)
    out, lse = _prefill(t, wl, api.SA_PREFILL_SPARSE, idx_out=idx)
    fi, fc, si, sc, _ = _select_both(t, wl.topk)
    gi = idx.cpu().numpy()
    assert np.array_equal(gi, fi)
    ro, rl = oracle.sparse_mla(wl.q_lat, wl.q_rope, wl.kv, gi, wl.sm_scale, dc=wl.dc)
    assert_attention_close(out, ro, ATTN_ATOL_BF16, lse, rl)


def test_prefill_sparse_mode_fp8_ragged():
    _announce("prefill sparse fp8 keys, spread q_pos, ragged kv_len")
    wl = workloads.prefill_batch(B=2, T=400, L=1500, HI=64, dI=128, topk=256, H=64, fp8=True,
                                 q_pos="spread", kv_len=[1500, 900])
    t = wl.to(DEV)
    idx = torch.empty((wl.B, wl.T, wl.topk), dtype=torch.int32, device=DEV)
    out, lse = _prefill(t, wl, api.SA_PREFILL_SPARSE, idx_out=idx)
    s = api.sparse_attn_indexer_scores(t.q_idx, t.w, t.k_idx, k_scale=t.k_scale, q_pos=t.q_pos,
                                       kv_len=t.kv_len)
    si, sc = api.sparse_attn_topk(s, wl.topk, q_pos=t.q_pos, kv_len=t.kv_len)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    assert np.array_equal(gi, si.cpu().numpy())
    oi, oc = oracle.topk(s.cpu().double().numpy(), wl.topk, q_pos=wl.q_pos, kv_len=wl.kv_len)
    assert np.array_equal(gi, oi)
    ro, rl = oracle.sparse_mla(wl.q_lat, wl.q_rope, wl.kv, gi, wl.sm_scale, dc=wl.dc)
    assert_attention_close(out, ro, ATTN_ATOL_BF16, lse, rl)


def _visible(wl):
    L = wl.L
    qp = wl.q_pos.numpy().astype(np.int64)
    lim = np.minimum(qp + 1, L)
    if wl.kv_len is not None:
        lim = np.minimum(lim, wl.kv_len.numpy()[:, None])
    return np.arange(L)[None, None, :] < lim[:, :, None]


@pytest.mark.parametrize("case", [dict(B=1, T=700, L=700, H=64),
                                  dict(B=2, T=300, L=2500, H=128, kv_len=[2500, 1900])],
                         ids=["causal700", "ragged_L2500"])
def test_prefill_dense_mode(case):
    _announce(f"prefill dense {case}")
    wl = workloads.prefill_batch(HI=64, dI=128, topk=64, **case)
    t = wl.to(DEV)
    out, lse = _prefill(t, wl, api.SA_PREFILL_DENSE)
    ro, rl = oracle.masked_mla(wl.q_lat, wl.q_rope, wl.kv, _visible(wl), wl.sm_scale, dc=wl.dc)
    assert_attention_close(out, ro, ATTN_ATOL_BF16, lse, rl)


def test_prefill_dense_mode_empty_rows():
    _announce("prefill dense empty rows")
    wl = workloads.prefill_batch(B=1, T=40, L=300, H=64, topk=16)
    wl.q_pos[0, :3] = -1
    t = wl.to(DEV)
    out, lse = _prefill(t, wl, api.SA_PREFILL_DENSE)
    assert torch.all(out[0, :3] == 0)
    assert torch.all(torch.isneginf(lse[0, :3]))
    vis = _visible(wl)[:, 3:]
    ro, rl = oracle.masked_mla(wl.q_lat[:, 3:], wl.q_rope[:, 3:], wl.kv, vis, wl.sm_scale,
                               dc=wl.dc)
    assert_attention_close(out[:, 3:], ro, ATTN_ATOL_BF16, lse[:, 3:], rl)


def test_prefill_auto_mode_picks_by_length():
    _announce("prefill auto: dense at L <= k, sparse above")
    short = workloads.prefill_batch(B=1, T=100, L=700, H=64, topk=700)
    t = short.to(DEV)
    a_out, a_lse = _prefill(t, short, api.SA_PREFILL_AUTO)
    d_out, d_lse = _prefill(t, short, api.SA_PREFILL_DENSE)
    assert torch.equal(a_out, d_out) and torch.equal(a_lse, d_lse)
    long = workloads.prefill_batch(B=1, T=64, L=701, H=64, topk=700)
    t = long.to(DEV)
    a_out, a_lse = _prefill(t, long, api.SA_PREFILL_AUTO)
    s_out, s_lse = _prefill(t, long, api.SA_PREFILL_SPARSE)
    assert torch.equal(a_out, s_out) and torch.equal(a_lse, s_lse)


def test_prefill_sparse_equals_dense_when_k_covers_every_row():
    # with k >= every row's candidate count the sparse set is every candidate
    _announce("prefill sparse == dense at k >= L")
    wl = workloads.prefill_batch(B=1, T=200, L=500, H=64, topk=512)
    t = wl.to(DEV)
    s_out, s_lse = _prefill(t, wl, api.SA_PREFILL_SPARSE)
    d_out, d_lse = _prefill(t, wl, api.SA_PREFILL_DENSE)
    torch.testing.assert_close(s_out, d_out, atol=2e-5, rtol=0)
    torch.testing.assert_close(s_lse, d_lse, atol=2e-5, rtol=0)


# --------------------------------------------------------------------------
# full size: prefill_16k (T = L = 16384, k = 2048)
# --------------------------------------------------------------------------

def test_prefill_select_fullsize():
    _announce("prefill_select full size T=L=16384 k=2048")
    wl = workloads.prefill_16k(with_mla=False)
    t = wl.to(DEV)
    fi, fc, si, sc, s = _select_both(t, wl.topk)
    # every row equals the staged indexer -> top-k path
    assert np.array_equal(fc, sc) and np.array_equal(fi, si)
    rows = [0, 1, 2046, 2047, 2048, 5000, 8191, 12000, 16383]
    sr = s[:, rows].cpu().double().numpy()
    qp = wl.q_pos[:, rows].contiguous()
    oi, oc = oracle.topk(sr, wl.topk, q_pos=qp)
    assert np.array_equal(fc[:, rows], oc) and np.array_equal(fi[:, rows], oi)
    del s
    torch.cuda.empty_cache()


def test_prefill_dense_fullsize_sampled():
    _announce("prefill dense full size L=16384, sampled queries")
    wl = workloads.prefill_16k(n_needles=0)
    t = wl.to(DEV)
    out, lse = _prefill(t, wl, api.SA_PREFILL_DENSE)
    rows = [0, 777, 16383]
    vis = _visible(wl)[:, rows]
    ro, rl = oracle.masked_mla(wl.q_lat[:, rows].contiguous(), wl.q_rope[:, rows].contiguous(),
                               wl.kv, vis, wl.sm_scale, dc=wl.dc)
    assert_attention_close(out[:, rows], ro, ATTN_ATOL_BF16, lse[:, rows], rl)


@pytest.mark.parametrize("B,T,L", [
    # rows above the fused select's 32768 positions: staged, in chunks of as
    # many query rows as 1 GiB of scores holds (4096 at L = 65536), so each
    # sequence runs 4096 + 104 rows
    (2, 4200, 65536),
    # staged where measured faster, one chunk of T rows: T >= 2048 with
    # L >= 2048, and T >= 1024 with L > 16384
    (1, 2100, 20000),
    (2, 2300, 3000),
    (1, 1100, 20000),
])
def test_prefill_sparse_staged_select(B, T, L):
    _announce(f"prefill sparse B={B} T={T} L={L} (staged select)")
    wl = workloads.prefill_batch(B=B, T=T, L=L, HI=64, dI=128, topk=2048, H=64)
    t = wl.to(DEV)
    idx = torch.empty((wl.B, wl.T, wl.topk), dtype=torch.int32, device=DEV)
    out, lse = _prefill(t, wl, api.SA_PREFILL_SPARSE, idx_out=idx)
    s = api.sparse_attn_indexer_scores(t.q_idx, t.w, t.k_idx, q_pos=t.q_pos)
    si, sc = api.sparse_attn_topk(s, wl.topk, q_pos=t.q_pos)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    assert np.array_equal(gi, si.cpu().numpy())
    rows = sorted({0, min(4095, T - 1), min(4096, T - 1), T - 1})
    sr = s[:, rows].cpu().double().numpy()
    oi, oc = oracle.topk(sr, wl.topk, q_pos=wl.q_pos[:, rows].contiguous())
    assert np.array_equal(gi[:, rows], oi)
    del s
    ro, rl = oracle.sparse_mla(wl.q_lat[:, rows].contiguous(), wl.q_rope[:, rows].contiguous(),
                               wl.kv, gi[:, rows], wl.sm_scale, dc=wl.dc)
    assert_attention_close(out[:, rows], ro, ATTN_ATOL_BF16, lse[:, rows], rl)
