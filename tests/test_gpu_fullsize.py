"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times, checked against the oracle on sampled outputs.

* decode, B=32, L=32768, bf16 (the benchmark step): the fused decode over the
  whole batch against the staged entry points over the whole batch:
  identical index sets, outputs equal (checked up to the rounding of a
  different KV split, which the fused path is free to choose).  Sampled sequences of the fused outputs
  are checked end to end against the oracle: every index score of the
  sequence, the selected set, and the attention output of all 128 heads given
  the GPU's indices.
* decode, B=8, L=131072, fp8 indexer keys with per-token scales: the same, on
  the long-row top-k path (chunked select + merge).
* causal prefill, T=L=16384: indexer (MFMA prefill kernel) and top-k over all
  16384 query rows; sampled rows (first, last, needle-aligned, and spread
  ones) checked against the oracle, and the sparse MLA of the sampled rows
  given the GPU's indices.

The oracle computes only the sampled sequences / rows, so each test takes
seconds of CPU time.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from top_indexer_sparse_amd import api, workloads

from parity import (ATTN_ATOL_BF16, ATTN_ATOL_FP8, assert_attention_close,
                    assert_index_sets, assert_scores_close, score_floor)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _announce(msg):
    print(f"\n[fullsize] {msg}", file=sys.stderr, flush=True)


def _decode_full(wl, seqs, attn_atol):
    t = wl.to(DEV)
    dc = wl.dc
    c_kv, k_rope = t.kv[..., :dc], t.kv[..., dc:]
    # staged entry points over the whole batch
    s = api.sparse_attn_indexer_scores(t.q_idx, t.w, t.k_idx, k_scale=t.k_scale,
                                       kv_len=t.kv_len)
    idx, cnt = api.sparse_attn_topk(s, wl.topk, kv_len=t.kv_len)
    out, lse = api.sparse_attn_mla_forward(t.q_lat, t.q_rope, c_kv, k_rope, idx, wl.sm_scale)
    # the fused decode (what the benchmark times) over the same batch
    out2, lse2, idx2 = api.sparse_attn_decode(t.q_idx, t.w, t.k_idx, t.k_scale, t.kv_len,
                                              wl.topk, t.q_lat, t.q_rope, c_kv, k_rope,
                                              wl.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2), "fused and staged index sets differ"
    # the halves may split the index range over a different number of
    # work-groups, i.e. other softmax reference maxima and another merge: the
    # same result up to the rounding of the bf16 hi+lo weights (~2^-17 relative)
    d_out = ((out - out2).abs() - 2e-5 * out.abs()).max().item()
    d_lse = (lse - lse2).abs().max().item()
    assert d_out <= 1e-4, f"fused and staged outputs differ: {d_out:.3g}"
    assert d_lse <= 1e-4, f"fused and staged lse differ: {d_lse:.3g}"
    out, lse = out2, lse2
    for b in seqs:
        _announce(f"{wl.name}: oracle on sequence {b}")
        sub = wl.slice_batch(b, b + 1)
        rs = oracle.indexer(sub.q_idx, sub.w, sub.k_idx, k_scale=sub.k_scale, kv_len=sub.kv_len)
        kdeq = oracle.dequantized_keys(sub.k_idx, sub.k_scale)
        assert_scores_close(s[b:b + 1], rs, score_floor(sub.q_idx, sub.w, kdeq))
        oi, oc = oracle.topk(rs, wl.topk, kv_len=sub.kv_len)
        gi = idx[b:b + 1].cpu().numpy()
        assert_index_sets(gi, cnt[b:b + 1], oi, oc, rs)
        ro, rl = oracle.sparse_mla(sub.q_lat, sub.q_rope, sub.kv, gi, wl.sm_scale, dc=dc)
        assert_attention_close(out[b:b + 1], ro, attn_atol, lse[b:b + 1], rl)
        if wl.needles is not None:  # sanity, not parity: planted rows are selected
            assert set(wl.needles[b].tolist()) <= set(gi[0, 0].tolist())


def test_fullsize_decode_32k():
    _announce("decode B=32 L=32768 k=2048 bf16")
    wl = workloads.decode_32k()
    _decode_full(wl, seqs=[0, 13, 31], attn_atol=ATTN_ATOL_BF16)


def test_decode_64_sequences_1024_positions_per_wave():
    # 64 rows of 32768 positions fill the score kernel's 512 work-groups at
    # its longest span, 1024 positions (64 chunks) per wave, and a candidate
    # list of 4096 slots per work-group; the batch above runs 512 per wave
    _announce("decode B=64 L=32768 k=2048 bf16 (1024 positions per wave)")
    wl = workloads.decode_32k(B=64)
    _decode_full(wl, seqs=[0, 37, 63], attn_atol=ATTN_ATOL_BF16)


def test_fullsize_decode_128k_fp8():
    _announce("decode B=8 L=131072 k=2048 fp8 keys")
    wl = workloads.decode_128k_fp8()
    # the MLA inputs are bf16 here too; the fp8 bound covers the indexer side
    _decode_full(wl, seqs=[0, 5], attn_atol=ATTN_ATOL_BF16)


def test_fullsize_prefill_16k():
    _announce("prefill T=L=16384 k=2048 bf16")
    wl = workloads.prefill_16k()
    t = wl.to(DEV)
    T = wl.T
    s = api.sparse_attn_indexer_scores(t.q_idx, t.w, t.k_idx, q_pos=t.q_pos)
    idx, cnt = api.sparse_attn_topk(s, wl.topk, q_pos=t.q_pos)
    torch.cuda.synchronize()
    rows = sorted({0, 1, 7, 2047, 2048, 4095, 8191, 12345, T - 2, T - 1})
    sel = torch.tensor(rows, dtype=torch.long)
    q_idx, w, q_pos = wl.q_idx[:, sel], wl.w[:, sel], wl.q_pos[:, sel]
    _announce(f"prefill: oracle on rows {rows}")
    rs = oracle.indexer(q_idx, w, wl.k_idx, q_pos=q_pos)
    g_s = s[:, sel.to(DEV)]
    assert_scores_close(g_s, rs, score_floor(q_idx, w, oracle.decode(wl.k_idx)))
    oi, oc = oracle.topk(rs, wl.topk, q_pos=q_pos)
    gi = idx[:, sel.to(DEV)].cpu().numpy()
    assert_index_sets(gi, cnt[:, sel.to(DEV)], oi, oc, rs)
    # sparse MLA on the sampled rows, given the GPU's indices
    tq = t.q_lat[:, sel.to(DEV)].contiguous()
    tr = t.q_rope[:, sel.to(DEV)].contiguous()
    gidx = idx[:, sel.to(DEV)].contiguous()
    out, lse = api.sparse_attn_mla_forward(tq, tr, t.kv[..., :wl.dc], t.kv[..., wl.dc:], gidx,
                                           wl.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_mla(wl.q_lat[:, sel], wl.q_rope[:, sel], wl.kv, gi, wl.sm_scale,
                               dc=wl.dc)
    assert_attention_close(out, ro, ATTN_ATOL_BF16, lse, rl)
    # the last query sees every needle
    assert set(wl.needles[0].tolist()) <= set(gi[0, -1].tolist())
