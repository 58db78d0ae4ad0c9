"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Sizes the oracle finishes in seconds, spanning several tiles and a ragged
tail, plus edge cases (ragged kv_len, empty rows, k above the candidate
count, ties).  Full-size workloads are in test_gpu_fullsize.py.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from top_indexer_sparse_amd import api, workloads
from parity import (ATTN_ATOL_BF16, assert_attention_close, assert_index_sets,
                    assert_scores_close, score_floor)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _cuda(*ts):
    return [None if t is None else t.to(DEV) for t in ts]


def _announce(msg):
    print(f"[case] {msg}", flush=True)


# --------------------------------------------------------------------------
# indexer
# --------------------------------------------------------------------------

def test_indexer_exact_small_integers():
    wl = workloads.tiny_prefill()
    _announce("indexer tiny_prefill fp32 L=1024")
    q, w, k, qp = _cuda(wl.q_idx, wl.w, wl.k_idx, wl.q_pos)
    g = api.sparse_attn_indexer_scores(q, w, k, q_pos=qp)
    torch.cuda.synchronize()
    ref = oracle.indexer(wl.q_idx, wl.w, wl.k_idx, q_pos=wl.q_pos)
    assert np.array_equal(g.cpu().double().numpy(), ref)  # bit-exact


@pytest.mark.parametrize("HI,dI,fp8", [(64, 128, False), (16, 128, False), (32, 64, False),
                                       (128, 128, False), (64, 128, True), (16, 64, True)])
def test_indexer_mfma_decode(HI, dI, fp8):
    _announce(f"indexer decode HI={HI} dI={dI} fp8={fp8}")
    B, L = 3, 3001
    kv_len = [3001, 1777, 5]
    if fp8:
        wl = workloads.decode_128k_fp8(B=B, L=L, HI=HI, dI=dI, H=64, boost_frac=0.02)
        wl.kv_len = torch.tensor(kv_len, dtype=torch.int32)
    else:
        wl = workloads.decode_32k(B=B, L=L, HI=HI, dI=dI, H=64, kv_len=kv_len, n_needles=4)
    q, w, k, ks, kl = _cuda(wl.q_idx, wl.w, wl.k_idx, wl.k_scale, wl.kv_len)
    g = api.sparse_attn_indexer_scores(q, w, k, k_scale=ks, kv_len=kl)
    torch.cuda.synchronize()
    ref = oracle.indexer(wl.q_idx, wl.w, wl.k_idx, k_scale=wl.k_scale, kv_len=wl.kv_len)
    fl = score_floor(wl.q_idx, wl.w, oracle.dequantized_keys(wl.k_idx, wl.k_scale))
    assert_scores_close(g, ref, fl)


@pytest.mark.parametrize("HI,dI,fp8", [(64, 128, False), (128, 128, False), (64, 128, True),
                                       (16, 64, True), (32, 64, False)])
def test_decode_and_prefill_score_kernels_carry_the_same_bits(HI, dI, fp8):
    # The decode score kernel (one query per row; keys and, where it fits, the
    # query block staged through LDS) and the staged prefill score kernel (eight
    # queries sharing LDS key tiles) compute the same contraction in the same
    # order, so every score must match bit for bit.  L = 700 leaves ragged
    # tails of both kernels' chunks and tiles.
    _announce(f"indexer decode vs prefill bits HI={HI} dI={dI} fp8={fp8}")
    B, T, L = 2, 8, 700
    gen = torch.Generator().manual_seed(1000 * HI + dI + int(fp8))
    q = torch.randn((B, T, HI, dI), generator=gen).to(torch.bfloat16)
    w = torch.rand((B, T, HI), generator=gen)
    k = torch.randn((B, L, dI), generator=gen)
    ks = None
    if fp8:
        k = k.to(torch.float8_e4m3fn)
        ks = 0.5 + torch.rand((B, L), generator=gen)
    else:
        k = k.to(torch.bfloat16)
    q, w, k, ks = _cuda(q, w, k, ks)
    qp = torch.full((B, T), L - 1, dtype=torch.int32, device=DEV)  # every position a candidate
    pre = api.sparse_attn_indexer_scores(q, w, k, k_scale=ks, q_pos=qp)
    dec = torch.cat([api.sparse_attn_indexer_scores(q[:, t:t + 1].contiguous(),
                                                    w[:, t:t + 1].contiguous(), k, k_scale=ks)
                     for t in range(T)], dim=1)
    torch.cuda.synchronize()
    assert torch.isfinite(pre).all()
    assert torch.equal(pre.view(torch.int32), dec.view(torch.int32)), "score bits differ"


@pytest.mark.parametrize("fp8,dI", [(False, 128), (True, 128), (False, 64), (True, 64)])
def test_indexer_mfma_prefill(fp8, dI):
    # the staged score kernel's key tiles: 16, 8, 8 and 4 KB per 64 positions
    # (every wave, or only the first four, issues a 1 KB copy per block)
    _announce(f"indexer prefill L=520 fp8={fp8} dI={dI}")
    L = 520
    wl = workloads.prefill_16k(L=L, dI=dI, with_mla=False, n_needles=0)
    k_idx, k_scale = wl.k_idx, None
    if fp8:
        k32 = wl.k_idx.float()
        k_scale = k32.abs().amax(-1) / 448.0
        k_idx = (k32 / k_scale[..., None]).to(torch.float8_e4m3fn)
    # a second sequence with a shorter cache exercises kv_len with q_pos
    q_idx = torch.cat([wl.q_idx, wl.q_idx.flip(1)])
    w = torch.cat([wl.w, wl.w.flip(1)])
    k_idx = torch.cat([k_idx, k_idx.flip(1)])
    k_scale = None if k_scale is None else torch.cat([k_scale, k_scale.flip(1)])
    q_pos = torch.cat([wl.q_pos, wl.q_pos])
    kv_len = torch.tensor([L, 301], dtype=torch.int32)
    q, ww, k, ks, qp, kl = _cuda(q_idx, w, k_idx, k_scale, q_pos, kv_len)
    g = api.sparse_attn_indexer_scores(q, ww, k, k_scale=ks, q_pos=qp, kv_len=kl)
    torch.cuda.synchronize()
    ref = oracle.indexer(q_idx, w, k_idx, k_scale=k_scale, q_pos=q_pos, kv_len=kv_len)
    fl = score_floor(q_idx, w, oracle.dequantized_keys(k_idx, k_scale))
    assert_scores_close(g, ref, fl)


@pytest.mark.parametrize("T", [1, 16])
def test_indexer_mfma_relu_maps_nan_products_to_zero(T):
    # The MFMA score kernels take ReLU(x) as the median of x, 0 and +inf:
    # a NaN head product contributes 0, as fmaxf(x, 0) would.  A key row
    # with NaN elements then scores exactly 0, and every other position
    # scores what it scores with that row zeroed (the oracle's input, which
    # must be finite).  T = 1 runs the decode kernel, T = 16 with q_pos the
    # staged prefill kernel and the fused prefill select.
    _announce(f"indexer NaN key rows T={T}")
    g0 = torch.Generator().manual_seed(41)
    B, HI, dI, L = 2, 64, 128, 700
    q = torch.randn(B, T, HI, dI, generator=g0).to(torch.bfloat16)
    w = torch.rand(B, T, HI, generator=g0) - 0.2
    k = torch.randn(B, L, dI, generator=g0).to(torch.bfloat16)
    bad = [3, 64, 65, 333, 683]  # candidates of every query (q_pos >= L - T)
    k_nan = k.clone()
    k_nan[0, bad] = float("nan")
    k_nan[1, bad, 7] = float("nan")  # one NaN element per row
    k_zero = k.clone()
    k_zero[:, bad] = 0
    qp = None if T == 1 else torch.arange(L - T, L, dtype=torch.int32).repeat(B, 1)
    gq, gw, gk, gqp = _cuda(q, w, k_nan, qp)
    g = api.sparse_attn_indexer_scores(gq, gw, gk, q_pos=gqp)
    torch.cuda.synchronize()
    gs = g.cpu()
    assert (gs[:, :, bad] == 0).all().item()
    ref = oracle.indexer(q, w, k_zero, q_pos=qp)
    assert_scores_close(g, ref, score_floor(q, w, oracle.decode(k_zero)))
    if T > 1:  # the fused select scores with the same arithmetic
        idx, cnt = api.sparse_attn_prefill_select(gq, gw, gk, 64, q_pos=gqp)
        torch.cuda.synchronize()
        oi, oc = oracle.topk(gs.double().numpy(), 64, q_pos=qp)
        assert np.array_equal(idx.cpu().numpy(), oi)


def test_indexer_vector_path_bf16_odd_heads():
    _announce("indexer vector path HI=12 bf16")
    g0 = torch.Generator().manual_seed(5)
    B, T, HI, dI, L = 2, 3, 12, 64, 257
    q = torch.randn(B, T, HI, dI, generator=g0).to(torch.bfloat16)
    w = torch.rand(B, T, HI, generator=g0) - 0.3  # negative weights are allowed
    k = torch.randn(B, L, dI, generator=g0).to(torch.bfloat16)
    qp = torch.tensor([[0, 100, 256], [5, 6, 300]], dtype=torch.int32)
    gq, gw, gk, gqp = _cuda(q, w, k, qp)
    g = api.sparse_attn_indexer_scores(gq, gw, gk, q_pos=gqp)
    torch.cuda.synchronize()
    ref = oracle.indexer(q, w, k, q_pos=qp)
    assert_scores_close(g, ref, score_floor(q, w, oracle.decode(k)))


# --------------------------------------------------------------------------
# top-k (same scores on both sides -> identical sets)
# --------------------------------------------------------------------------

def _topk_both(scores, k, q_pos=None, kv_len=None):
    gi, gc = api.sparse_attn_topk(*_cuda(scores), k, *_cuda(q_pos, kv_len))
    torch.cuda.synchronize()
    oi, oc = oracle.topk(scores.double().numpy(), k, q_pos=q_pos, kv_len=kv_len)
    return gi.cpu().numpy(), gc.cpu().numpy(), oi, oc


def test_topk_exact_small_integer_workload():
    _announce("topk tiny_prefill k=64 (many ties)")
    wl = workloads.tiny_prefill()
    s = torch.from_numpy(oracle.indexer(wl.q_idx, wl.w, wl.k_idx, q_pos=wl.q_pos)).float()
    gi, gc, oi, oc = _topk_both(s, 64, q_pos=wl.q_pos)
    assert np.array_equal(gc, oc) and np.array_equal(gi, oi)


# Few rows of length >= 8192 take the split path (chunk work-groups + one
# select work-group per row, with a fallback from the row itself); the other
# shapes and the many-row cases take one work-group per row (chunks and a merge
# beyond 32768 positions).
@pytest.mark.parametrize("L,k,kind,B", [(5000, 2048, "normal", 3), (32768, 2048, "ties", 3),
                                        (32768, 4096, "signed", 3), (1000, 1, "ties", 3),
                                        (70000, 2048, "ties", 3), (131072, 2048, "normal", 3),
                                        (40000, 64, "zeros", 3), (70000, 2048, "narrow", 3),
                                        (70000, 2048, "allequal", 3), (32768, 2048, "hidden", 3),
                                        (12345, 300, "normal", 3), (40000, 512, "ties", 130)])
def test_topk_matches_oracle_bitexact(L, k, kind, B):
    _announce(f"topk L={L} k={k} {kind} rows={B}")
    g0 = torch.Generator().manual_seed(L + k)
    if kind == "hidden":
        # the largest scores sit on positions the row sample never visits
        s = torch.rand(B, 1, L, generator=g0)
        s[:, :, 1::16] += 10.0
    elif kind == "normal":
        s = torch.randn(B, 1, L, generator=g0).abs()
    elif kind == "ties":
        s = torch.randint(0, 40, (B, 1, L), generator=g0).float() * 0.25
    elif kind == "narrow":
        # every key shares its top 11 bits: the first bin exceeds what LDS holds
        s = 1.0 + torch.randint(0, 1024, (B, 1, L), generator=g0).float() * 2.0 ** -20
    elif kind == "allequal":
        s = torch.full((B, 1, L), 3.0)
    elif kind == "zeros":
        s = torch.zeros(B, 1, L)
        s[:, :, ::97] = 1.0
        s[:, :, 1::5] = -0.0
    else:
        s = torch.randn(B, 1, L, generator=g0) * 1e3
        s[:, :, ::7] = -s[:, :, ::7].abs()
    kv_len = torch.tensor([L, L // 2 + 3, min(k, L) - 1 if min(k, L) > 1 else 1] * (B // 3) +
                          [L] * (B % 3), dtype=torch.int32)
    gi, gc, oi, oc = _topk_both(s, k, kv_len=kv_len)
    assert np.array_equal(gc, oc)
    assert np.array_equal(gi, oi)


def test_topk_causal_rows_and_empty():
    _announce("topk causal rows, empty rows")
    g0 = torch.Generator().manual_seed(9)
    T, L, k = 70, 200, 16
    s = torch.randn(2, T, L, generator=g0)
    q_pos = torch.arange(T, dtype=torch.int32).repeat(2, 1)
    q_pos[1, :5] = -1  # queries with no candidate
    kv_len = torch.tensor([L, 0], dtype=torch.int32)
    gi, gc, oi, oc = _topk_both(s, k, q_pos=q_pos, kv_len=kv_len)
    assert np.array_equal(gc, oc) and np.array_equal(gi, oi)
    assert np.all(gc[1] == 0) and np.all(gi[1] == -1)


def test_topk_excludes_nan_and_neg_inf():
    # documented GPU behaviour: NaN and -inf scores are never selected
    _announce("topk NaN/-inf exclusion")
    s = torch.tensor([[[1.0, float("nan"), 3.0, float("-inf"), 2.0, float("inf")]]])
    gi, gc = api.sparse_attn_topk(s.to(DEV), 4)
    torch.cuda.synchronize()
    assert gc.item() == 4
    assert gi.cpu().tolist() == [[[0, 2, 4, 5]]]


# --------------------------------------------------------------------------
# sparse MLA given identical indices
# --------------------------------------------------------------------------

def test_mla_fp32_vector_path():
    _announce("mla fp32 tiny_prefill dims")
    wl = workloads.tiny_prefill(L=300, topk=64)
    s = oracle.indexer(wl.q_idx, wl.w, wl.k_idx, q_pos=wl.q_pos)
    oi, oc = oracle.topk(s, wl.topk, q_pos=wl.q_pos)
    ql, qr, kv, idx = _cuda(wl.q_lat, wl.q_rope, wl.kv, torch.from_numpy(oi))
    out, lse = api.sparse_attn_mla_forward(ql, qr, kv[..., :wl.dc], kv[..., wl.dc:], idx,
                                           wl.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_mla(wl.q_lat, wl.q_rope, wl.kv, oi, wl.sm_scale, dc=wl.dc)
    err = assert_attention_close(out, ro, 2e-3, lse, rl)
    assert err < 1e-4  # fp32 arithmetic


# KV splits per (query, 64-head group): 32, 4, 2 and 8 -- the split combine's
# general path and its load-first paths for up to 4 and 8 splits
@pytest.mark.parametrize("B,k,H", [(2, 2048, 128), (5, 300, 64), (40, 96, 128), (16, 600, 128)])
def test_mla_bf16_mfma(B, k, H):
    _announce(f"mla bf16 B={B} k={k} H={H}")
    L = 2600
    wl = workloads.decode_32k(B=B, L=L, H=H, n_needles=16 if B < 10 else 0)
    rng = np.random.default_rng(B * 1000 + k)
    idx = np.stack([np.sort(rng.choice(L, k, replace=False)) for _ in range(B)])[:, None]
    idx = idx.astype(np.int32)
    if wl.needles is not None:  # put the needles in the set (duplicates count twice)
        for b in range(B):
            idx[b, 0, :16] = wl.needles[b].numpy()
    idx[0, 0, -7:] = -1          # padding slots are skipped
    idx[-1, 0, 3] = L + 5        # out-of-range slot is skipped
    ql, qr, kv, gidx = _cuda(wl.q_lat, wl.q_rope, wl.kv, torch.from_numpy(idx))
    out, lse = api.sparse_attn_mla_forward(ql, qr, kv[..., :wl.dc], kv[..., wl.dc:], gidx,
                                           wl.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_mla(wl.q_lat, wl.q_rope, wl.kv, idx, wl.sm_scale, dc=wl.dc)
    assert_attention_close(out, ro, ATTN_ATOL_BF16, lse, rl)


def test_mla_empty_rows_give_zero_and_neg_inf():
    _announce("mla empty rows")
    wl = workloads.decode_32k(B=2, L=300, H=64, n_needles=0)
    idx = np.full((2, 1, 64), -1, dtype=np.int32)
    idx[1, 0, :10] = np.arange(10)
    ql, qr, kv, gidx = _cuda(wl.q_lat, wl.q_rope, wl.kv, torch.from_numpy(idx))
    out, lse = api.sparse_attn_mla_forward(ql, qr, kv[..., :wl.dc], kv[..., wl.dc:], gidx,
                                           wl.sm_scale)
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    ro, rl = oracle.sparse_mla(wl.q_lat[1:], wl.q_rope[1:], wl.kv[1:], idx[1:], wl.sm_scale,
                               dc=wl.dc)
    assert_attention_close(out[1:], ro, ATTN_ATOL_BF16, lse[1:], rl)


def test_mla_separate_cache_tensors_fp32_rope_stride():
    # c_kv and k_rope as two separate tensors (different row strides)
    _announce("mla separate caches")
    g0 = torch.Generator().manual_seed(3)
    B, T, H, dc, dR, L, k = 2, 2, 8, 128, 32, 90, 40
    ql = torch.randn(B, T, H, dc, generator=g0)
    qr = torch.randn(B, T, H, dR, generator=g0)
    c = torch.randn(B, L, dc, generator=g0)
    r = torch.randn(B, L, dR, generator=g0)
    idx = torch.stack([torch.stack([torch.randperm(L, generator=g0)[:k] for _ in range(T)])
                       for _ in range(B)]).to(torch.int32)
    out, lse = api.sparse_attn_mla_forward(*_cuda(ql, qr, c, r, idx), 0.1)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_mla(ql, qr, c, idx.numpy(), 0.1, dc=dc, k_rope=r)
    assert_attention_close(out, ro, 1e-4, lse, rl)


# --------------------------------------------------------------------------
# fused decode and the whole path
# --------------------------------------------------------------------------

def test_fused_decode_small():
    _announce("fused decode B=4 L=5000 k=2048")
    B, L = 4, 5000
    wl = workloads.decode_32k(B=B, L=L, kv_len=[5000, 4000, 2100, 1500])
    t = wl.to(DEV)
    out, lse, idx = api.sparse_attn_decode(t.q_idx, t.w, t.k_idx, None, t.kv_len, wl.topk,
                                           t.q_lat, t.q_rope, t.kv[..., :wl.dc],
                                           t.kv[..., wl.dc:], wl.sm_scale)
    torch.cuda.synchronize()
    s = oracle.indexer(wl.q_idx, wl.w, wl.k_idx, kv_len=wl.kv_len)
    oi, oc = oracle.topk(s, wl.topk, kv_len=wl.kv_len)
    gi = idx.cpu().numpy()
    gc = (gi >= 0).sum(-1)
    assert_index_sets(gi, gc, oi, oc, s)
    # needles are found (sanity, not parity)
    for b in range(B):
        assert set(wl.needles[b].tolist()) <= set(gi[b, 0].tolist())
    ro, rl = oracle.sparse_mla(wl.q_lat, wl.q_rope, wl.kv, gi, wl.sm_scale, dc=wl.dc)
    assert_attention_close(out, ro, ATTN_ATOL_BF16, lse, rl)


def test_staged_path_equals_fused_decode():
    _announce("staged == fused decode")
    B, L = 3, 4100
    wl = workloads.decode_32k(B=B, L=L)
    t = wl.to(DEV)
    s = api.sparse_attn_indexer_scores(t.q_idx, t.w, t.k_idx)
    idx, cnt = api.sparse_attn_topk(s, wl.topk)
    out, lse = api.sparse_attn_mla_forward(t.q_lat, t.q_rope, t.kv[..., :wl.dc],
                                           t.kv[..., wl.dc:], idx, wl.sm_scale)
    out2, lse2, idx2 = api.sparse_attn_decode(t.q_idx, t.w, t.k_idx, None, None, wl.topk,
                                              t.q_lat, t.q_rope, t.kv[..., :wl.dc],
                                              t.kv[..., wl.dc:], wl.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_fused_decode_ragged_batch():
    """Fused decode over B=10 sequences with ragged kv_len (down to one valid
    position): index sets equal the staged path's, outputs match the oracle,
    and work queued right after it on the caller's stream sees the result."""
    _announce("fused decode: B=10 L=4100 ragged kv_len")
    B, L = 10, 4100
    kv_len = [4100, 4000, 3000, 2100, 2048, 2047, 100, 4100, 1, 3333]
    wl = workloads.decode_32k(B=B, L=L, kv_len=kv_len)
    t = wl.to(DEV)
    c_kv, k_rope = t.kv[..., :wl.dc], t.kv[..., wl.dc:]
    s = api.sparse_attn_indexer_scores(t.q_idx, t.w, t.k_idx, kv_len=t.kv_len)
    idx, cnt = api.sparse_attn_topk(s, wl.topk, kv_len=t.kv_len)
    out2, lse2, idx2 = api.sparse_attn_decode(t.q_idx, t.w, t.k_idx, None, t.kv_len, wl.topk,
                                              t.q_lat, t.q_rope, c_kv, k_rope, wl.sm_scale)
    # consume on the caller's stream right away: ordering is the library's job
    total = out2.abs().sum() + lse2.nan_to_num(neginf=0.0).abs().sum()
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    assert torch.isfinite(total).item()
    ro, rl = oracle.sparse_mla(wl.q_lat, wl.q_rope, wl.kv, idx2.cpu().numpy(), wl.sm_scale,
                               dc=wl.dc)
    assert_attention_close(out2, ro, ATTN_ATOL_BF16, lse2, rl)
    rs = oracle.indexer(wl.q_idx, wl.w, wl.k_idx, kv_len=wl.kv_len)
    oi, oc = oracle.topk(rs, wl.topk, kv_len=wl.kv_len)
    gi = idx2.cpu().numpy()
    assert_index_sets(gi, (gi >= 0).sum(-1), oi, oc, rs)


def test_prefill_path_small_causal():
    _announce("prefill path L=200 H=64")
    L = 200
    wl = workloads.prefill_16k(L=L, H=64, topk=64)
    t = wl.to(DEV)
    s = api.sparse_attn_indexer_scores(t.q_idx, t.w, t.k_idx, q_pos=t.q_pos)
    idx, cnt = api.sparse_attn_topk(s, wl.topk, q_pos=t.q_pos)
    out, lse = api.sparse_attn_mla_forward(t.q_lat, t.q_rope, t.kv[..., :wl.dc],
                                           t.kv[..., wl.dc:], idx, wl.sm_scale)
    torch.cuda.synchronize()
    rs = oracle.indexer(wl.q_idx, wl.w, wl.k_idx, q_pos=wl.q_pos)
    oi, oc = oracle.topk(rs, wl.topk, q_pos=wl.q_pos)
    assert_index_sets(idx.cpu().numpy(), cnt.cpu().numpy(), oi, oc, rs)
    gi = idx.cpu().numpy()
    ro, rl = oracle.sparse_mla(wl.q_lat, wl.q_rope, wl.kv, gi, wl.sm_scale, dc=wl.dc)
    assert_attention_close(out, ro, ATTN_ATOL_BF16, lse, rl)
    # causality: no selected position after its query
    for t_ in range(L):
        sel = gi[0, t_][gi[0, t_] >= 0]
        assert sel.max() <= t_


@pytest.mark.parametrize("order", ["ascending", "descending", "zigzag"])
def test_mla_bf16_score_ramps(order):
    # Scores that climb (or fall, or alternate) across the tiles of a split, so
    # the running maximum moves many times, by steps both inside and beyond the
    # kernel's rescaling margin; dynamic range ~80 in natural-log units.
    _announce(f"mla bf16 score ramp {order}")
    B, L, k, H = 2, 2100, 2048, 64
    wl = workloads.decode_32k(B=B, L=L, H=H, n_needles=0)
    kv = wl.kv.float()
    qr = wl.q_rope.float()
    ramp = torch.linspace(-40.0, 40.0, L)
    if order == "descending":
        ramp = ramp.flip(0)
    elif order == "zigzag":
        ramp = ramp * torch.where(torch.arange(L) % 3 == 0, 1.0, -0.5)
    for b in range(B):
        u = qr[b, 0].sum(0)
        u = u / u.norm()
        # k_rope_j = c_j * u  =>  q_rope_h . k_rope_j = c_j (q_rope_h . u)
        kv[b, :, wl.dc:] = ramp[:, None] * u[None, :] * (24.0 / max(float((qr[b, 0] @ u).abs().mean()), 1e-3))
    wl.kv = kv.to(torch.bfloat16)
    idx = np.stack([np.arange(k) for _ in range(B)])[:, None].astype(np.int32)
    ql, qrg, kvg, gidx = _cuda(wl.q_lat, wl.q_rope, wl.kv, torch.from_numpy(idx))
    out, lse = api.sparse_attn_mla_forward(ql, qrg, kvg[..., :wl.dc], kvg[..., wl.dc:], gidx,
                                           wl.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_mla(wl.q_lat, wl.q_rope, wl.kv, idx, wl.sm_scale, dc=wl.dc)
    assert_attention_close(out, ro, ATTN_ATOL_BF16, lse, rl, lse_atol=2e-3)
