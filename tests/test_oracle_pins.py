"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests re-types the oracle's formulas: each checks a printed
worked example, a closed form, an invariant the pages state, an independent
library routine (torch's casts, torch's scaled-dot-product attention, numpy's
dot), or brute force on tiny inputs.  A dropped term, a wrong sign or index or
a transposed operand in the oracle fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_examples.json")


@pytest.fixture(scope="module")
def ex():
    with open(GOLDEN) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# decoders: the bf16 layout and the OCP E4M3 definition, against torch's casts
# --------------------------------------------------------------------------

def test_bf16_decoder_all_codes(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = orc.decode_bf16_bits(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])


def test_e4m3fn_decoder_all_codes(orc):
    bits = np.arange(256, dtype=np.uint8)
    mine = orc.decode_e4m3fn_bits(bits)
    ref = torch.from_numpy(bits).view(torch.float8_e4m3fn).float().double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    # values fixed by the format definition
    assert mine[0x7E] == 448.0          # largest finite
    assert mine[0x01] == 2.0 ** -9      # smallest subnormal
    assert mine[0x08] == 2.0 ** -6      # smallest normal
    assert mine[0x38] == 1.0
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF])
    assert mine[0x80] == 0.0 and math.copysign(1.0, mine[0x80]) < 0
    assert np.isnan(mine).sum() == 2


# --------------------------------------------------------------------------
# lightning indexer
# --------------------------------------------------------------------------

def test_indexer_hand_example(orc):
    # two heads picking out the two coordinates, weights 1/2 and 2:
    # I_s = 1/2 * relu(k_s[0]) + 2 * relu(k_s[1])
    q = torch.tensor([[[[1.0, 0.0], [0.0, 1.0]]]])
    w = torch.tensor([[[0.5, 2.0]]])
    k = torch.tensor([[[3.0, -1.0], [-2.0, 4.0], [1.0, 1.0], [-1.0, -1.0]]])
    got = orc.indexer(q, w, k)
    assert got.tolist() == [[[1.5, 8.0, 2.5, 0.0]]]
    # causal bound s <= q_pos includes s = q_pos
    got = orc.indexer(q, w, k, q_pos=torch.tensor([[1]], dtype=torch.int32))
    assert got[0, 0, :2].tolist() == [1.5, 8.0]
    assert np.all(np.isneginf(got[0, 0, 2:]))
    # kv_len bound
    got = orc.indexer(q, w, k, kv_len=torch.tensor([3], dtype=torch.int32))
    assert got[0, 0, :3].tolist() == [1.5, 8.0, 2.5] and np.isneginf(got[0, 0, 3])


def test_indexer_single_head_is_relu_dot(orc):
    g = torch.Generator().manual_seed(1)
    q = torch.randn(2, 3, 1, 16, generator=g, dtype=torch.float64).float()
    k = torch.randn(2, 40, 16, generator=g, dtype=torch.float64).float()
    w = torch.ones(2, 3, 1)
    got = orc.indexer(q, w, k)
    qd, kd = q.double().numpy(), k.double().numpy()
    for b in range(2):
        for t in range(3):
            ref = np.maximum(kd[b] @ qd[b, t, 0], 0.0)
            np.testing.assert_allclose(got[b, t], ref, rtol=1e-13, atol=1e-13)


def test_indexer_homogeneity_and_head_additivity(orc):
    g = torch.Generator().manual_seed(2)
    B, T, HI, dI, L = 1, 2, 6, 8, 30
    q = torch.randn(B, T, HI, dI, generator=g)
    w = torch.rand(B, T, HI, generator=g)
    k = torch.randn(B, L, dI, generator=g)
    base = orc.indexer(q, w, k)
    # scaling keys by c > 0 scales the score (ReLU is positively homogeneous);
    # this is what lets a per-token fp8 scale be applied after the dot product
    np.testing.assert_allclose(orc.indexer(q, w, k * 4.0), 4.0 * base, rtol=1e-12)
    np.testing.assert_allclose(orc.indexer(q, w * 0.5, k), 0.5 * base, rtol=1e-12)
    # per-token scale through the fp8 path equals scaling those keys
    scale = torch.rand(B, L, generator=g) + 0.5
    np.testing.assert_allclose(orc.indexer(q, w, k, k_scale=scale),
                               base * scale.double().numpy()[:, None, :], rtol=1e-12)
    # the head sum splits over any partition of the heads
    a = orc.indexer(q[:, :, :2].contiguous(), w[:, :, :2].contiguous(), k)
    b = orc.indexer(q[:, :, 2:].contiguous(), w[:, :, 2:].contiguous(), k)
    np.testing.assert_allclose(a + b, base, rtol=1e-12, atol=1e-12)
    # negated query: relu zeroes the other half-space
    assert np.all(base >= 0)


def test_indexer_exact_integer_workload(orc):
    # small-integer workload: every score is a multiple of 1/4 and matches
    # an exact int64 evaluation (4*w is an integer)
    from top_indexer_sparse_amd import workloads
    wl = workloads.tiny_prefill(L=96, topk=8)
    got = orc.indexer(wl.q_idx, wl.w, wl.k_idx, q_pos=wl.q_pos)
    q = wl.q_idx.numpy().astype(np.int64)[0]
    k = wl.k_idx.numpy().astype(np.int64)[0]
    w4 = (wl.w.numpy() * 4).astype(np.int64)[0]
    dots = np.einsum("thi,si->ths", q, k)
    exact4 = (w4[:, :, None] * np.maximum(dots, 0)).sum(1)
    for t in range(wl.T):
        assert np.array_equal(got[0, t, :t + 1] * 4, exact4[t, :t + 1].astype(np.float64))
        assert np.all(np.isneginf(got[0, t, t + 1:]))


# --------------------------------------------------------------------------
# top-k
# --------------------------------------------------------------------------

def test_topk_page_example(orc, ex):
    e = ex["mis_selection"]
    idx, cnt = orc.topk(np.array([[e["index_scores"]]]), e["count"])
    assert idx[0, 0].tolist() == e["selected"] and cnt[0, 0] == 2


def test_topk_ties_go_to_lower_position(orc):
    idx, _ = orc.topk(np.array([[[5.0, 7.0, 7.0, 7.0, 1.0]]]), 2)
    assert idx[0, 0].tolist() == [1, 2]
    idx, _ = orc.topk(np.array([[[0.0, -0.0, 0.0]]]), 1)
    assert idx[0, 0].tolist() == [0]
    idx, _ = orc.topk(np.array([[[-0.0, 0.0, 3.0]]]), 2)
    assert idx[0, 0].tolist() == [0, 2]


def test_topk_brute_force_tiny(orc):
    # The top-k set is the k-subset with the largest score sum; among those
    # the lexicographically smallest (ties to lower positions).  Checked with
    # exact integer sums over every subset.
    rng = np.random.default_rng(3)
    for trial in range(60):
        L = int(rng.integers(1, 10))
        s = rng.integers(-3, 4, size=L)
        for k in range(1, L + 2):
            m = min(k, L)
            best = None
            for sub in itertools.combinations(range(L), m):
                key = (-int(s[list(sub)].sum()), sub)
                if best is None or key < best:
                    best = key
            idx, cnt = orc.topk(s.astype(np.float64)[None, None], k)
            assert cnt[0, 0] == m
            assert tuple(idx[0, 0, :m].tolist()) == best[1]
            assert np.all(idx[0, 0, m:] == -1)


def test_topk_fewer_candidates_and_causal(orc):
    s = np.arange(10, dtype=np.float64)[None, None].repeat(3, axis=1)
    q_pos = np.array([[0, 3, 9]], dtype=np.int32)
    idx, cnt = orc.topk(s, 5, q_pos=q_pos)
    assert cnt.tolist() == [[1, 4, 5]]
    assert idx[0, 0].tolist() == [0, -1, -1, -1, -1]
    assert idx[0, 1].tolist() == [0, 1, 2, 3, -1]
    assert idx[0, 2].tolist() == [5, 6, 7, 8, 9]
    idx, cnt = orc.topk(s[:, :1], 4, kv_len=np.array([0], dtype=np.int32))
    assert cnt[0, 0] == 0 and np.all(idx == -1)


def test_topk_rejects_nonfinite_candidates(orc):
    with pytest.raises(orc.OracleError):
        orc.topk(np.array([[[1.0, float("nan"), 0.0]]]), 1)
    # a non-finite value outside the candidate set is not looked at
    idx, _ = orc.topk(np.array([[[1.0, 2.0, float("nan")]]]), 1,
                      q_pos=np.array([[1]], dtype=np.int32))
    assert idx[0, 0].tolist() == [1]


# --------------------------------------------------------------------------
# sparse MLA
# --------------------------------------------------------------------------

def _mla_1q(orc, q_lat, q_rope, c, kr, idx, sm_scale=1.0, dense_mask=None):
    """One query, one head: helper building the [B,T,H,...] tensors."""
    q_lat = torch.tensor(q_lat, dtype=torch.float64).reshape(1, 1, 1, -1)
    c = np.asarray(c, dtype=np.float64)
    L, dc = c.shape
    if q_rope is None:
        kv = torch.tensor(c).reshape(1, L, dc)
        qr = torch.zeros(1, 1, 1, 0, dtype=torch.float64)
    else:
        kr = np.asarray(kr, dtype=np.float64).reshape(L, -1)
        kv = torch.tensor(np.concatenate([c, kr], axis=1)).reshape(1, L, -1)
        qr = torch.tensor(q_rope, dtype=torch.float64).reshape(1, 1, 1, -1)
    if dense_mask is not None:
        return orc.masked_mla(q_lat, qr, kv, np.asarray(dense_mask).reshape(1, 1, L),
                              sm_scale, dc=dc)
    ix = np.asarray(idx, dtype=np.int32).reshape(1, 1, -1)
    return orc.sparse_mla(q_lat, qr, kv, ix, sm_scale, dc=dc)


def test_absorbed_score_page_example(orc, ex):
    e = ex["absorbed_score"]
    UK = np.array(e["key_projection"])
    q = np.array(e["query"])
    c = np.array(e["latent"])
    assert (UK @ c).tolist() == e["key"]
    qt = UK.T @ q
    assert qt.tolist() == e["absorbed_query"]
    # a one-element set: softmax weight 1, lse equals the score itself
    _, lse = _mla_1q(orc, qt, None, [c], None, [0])
    assert lse[0, 0, 0] == e["score"]


def test_absorbed_score_random(orc):
    # q . (U_K c) == (U_K^T q) . c for random U_K, with a RoPE term added
    rng = np.random.default_rng(4)
    dq, dc, dR = 7, 5, 3
    UK = rng.standard_normal((dq, dc))
    q = rng.standard_normal(dq)
    qR = rng.standard_normal(dR)
    c = rng.standard_normal((1, dc))
    kR = rng.standard_normal((1, dR))
    _, lse = _mla_1q(orc, UK.T @ q, qR, c, kR, [0], sm_scale=0.37)
    direct = (float(np.dot(q, UK @ c[0])) + float(np.dot(qR, kR[0]))) * 0.37
    assert abs(lse[0, 0, 0] - direct) < 1e-12


def test_content_plus_position_page_example(orc, ex):
    e = ex["content_plus_position"]
    # q_lat = [1,0] and latent rows [1,0], [1,5]: both content scores 1, while
    # the rows' second coordinate (0 and 5) exposes the weights in the output.
    # RoPE: q^R = [1,0], k^R rows [0,0] and [2,0]: position scores 0 and 2.
    out, _ = _mla_1q(orc, [1.0, 0.0], [1.0, 0.0], [[1.0, 0.0], [1.0, 5.0]],
                     [[0.0, 0.0], [2.0, 0.0]], [0, 1],
                     sm_scale=1.0 / math.sqrt(e["total_dim"]))
    a2 = out[0, 0, 0, 1] / 5.0
    d = e["weights_decimals"]
    assert round(1.0 - a2, d) == e["weights"][0]
    assert round(a2, d) == e["weights"][1]
    assert abs(out[0, 0, 0, 0] - 1.0) < 1e-15


def _scalar_rows(values, scores):
    """Value v_j as a 1-d latent with content query 0; the score comes from a
    1-d RoPE term q^R = 1, k^R_j = score_j (sm_scale 1)."""
    c = [[v] for v in values]
    kr = [[s] for s in scores]
    return c, kr


def test_needle_page_example(orc, ex):
    e = ex["needle"]
    vals = [0.0] * e["length"]
    vals[e["needle_position"]] = e["needle_value"]
    c, kr = _scalar_rows(vals, [0.0] * e["length"])
    dense, _ = _mla_1q(orc, [0.0], [1.0], c, kr, None,
                       dense_mask=[1] * e["length"])
    assert dense[0, 0, 0, 0] == e["dense_output"]
    missed = [j for j in range(e["length"]) if j != e["needle_position"]]
    out, _ = _mla_1q(orc, [0.0], [1.0], c, kr, missed)
    assert out[0, 0, 0, 0] == e["missed_output"]


def test_mask_before_softmax_page_example(orc, ex):
    e = ex["mask_before_softmax"]
    for case in e["cases"]:
        c, kr = _scalar_rows(e["values"], case["scores"])
        out, _ = _mla_1q(orc, [0.0], [1.0], c, kr, None,
                         dense_mask=[int(v) for v in e["visible"]])
        assert out[0, 0, 0, 0] == case["output"]
        vis = [j for j, v in enumerate(e["visible"]) if v]
        out, _ = _mla_1q(orc, [0.0], [1.0], c, kr, vis)
        assert out[0, 0, 0, 0] == case["output"]


def test_mis_selection_page_example(orc, ex):
    e = ex["mis_selection"]
    idx, _ = orc.topk(np.array([[e["index_scores"]]]), e["count"])
    c, kr = _scalar_rows(e["values"], e["attention_scores"])
    n = len(e["values"])
    dense, _ = _mla_1q(orc, [0.0], [1.0], c, kr, None, dense_mask=[1] * n)
    assert dense[0, 0, 0, 0] > e["dense_output_greater_than"]
    # closed form 10 e^4 / (3 + e^4)
    assert abs(dense[0, 0, 0, 0] - 10 * math.exp(4) / (3 + math.exp(4))) < 1e-12
    sparse, _ = _mla_1q(orc, [0.0], [1.0], c, kr, idx[0, 0])
    assert sparse[0, 0, 0, 0] == e["sparse_output"]


def _rand_mla(seed, B=2, T=3, H=4, L=37, dc=6, dR=3):
    g = torch.Generator().manual_seed(seed)
    q_lat = torch.randn(B, T, H, dc, generator=g, dtype=torch.float64)
    q_rope = torch.randn(B, T, H, dR, generator=g, dtype=torch.float64)
    kv = torch.randn(B, L, dc + dR, generator=g, dtype=torch.float64)
    return q_lat, q_rope, kv


def test_mask_form_equals_gathered_form(orc):
    q_lat, q_rope, kv = _rand_mla(5)
    B, T, H, dc = q_lat.shape
    L = kv.shape[1]
    rng = np.random.default_rng(5)
    k = 9
    idx = np.stack([np.stack([np.sort(rng.choice(L, k, replace=False))
                              for _ in range(T)]) for _ in range(B)]).astype(np.int32)
    vis = np.zeros((B, T, L), dtype=np.uint8)
    for b in range(B):
        for t in range(T):
            vis[b, t, idx[b, t]] = 1
    o1, l1 = orc.sparse_mla(q_lat, q_rope, kv, idx, 0.3, dc=dc)
    o2, l2 = orc.masked_mla(q_lat, q_rope, kv, vis, 0.3, dc=dc)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=1e-12, atol=1e-12)


def test_full_selection_is_dense_attention_sdpa(orc):
    # k = L reproduces dense attention; dense attention checked against torch's
    # scaled_dot_product_attention in float64 (keys = [c, k^R], values = c)
    q_lat, q_rope, kv = _rand_mla(6, B=1, T=2, H=3, L=20, dc=5, dR=4)
    B, T, H, dc = q_lat.shape
    L = kv.shape[1]
    idx = np.tile(np.arange(L, dtype=np.int32), (B, T, 1))
    o, _ = orc.sparse_mla(q_lat, q_rope, kv, idx, 0.25, dc=dc)
    qfull = torch.cat([q_lat, q_rope], -1)            # [B,T,H,dc+dR]
    ref = torch.nn.functional.scaled_dot_product_attention(
        qfull.permute(0, 2, 1, 3),                    # [B,H,T,D]
        kv[:, None].expand(B, H, L, kv.shape[-1]),
        kv[:, None, :, :dc].expand(B, H, L, dc), scale=0.25)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-12, atol=1e-12)


def test_sparse_is_renormalised_dense(orc):
    # one-hot latent rows make the output equal to the weight vector itself;
    # the content query is zero so scores come from the RoPE term only
    L = 12
    rng = np.random.default_rng(7)
    scores = rng.standard_normal(L)
    c = np.eye(L)
    kr = scores[:, None]
    dense, _ = _mla_1q(orc, np.zeros(L), [1.0], c, kr, None, dense_mask=[1] * L)
    alpha = dense[0, 0, 0]
    np.testing.assert_allclose(alpha.sum(), 1.0, rtol=1e-14)
    S = [1, 4, 5, 9]
    sp, _ = _mla_1q(orc, np.zeros(L), [1.0], c, kr, S)
    Z = alpha[S].sum()
    expect = np.zeros(L)
    expect[S] = alpha[S] / Z
    np.testing.assert_allclose(sp[0, 0, 0], expect, rtol=1e-13, atol=1e-16)


def test_error_bound(orc):
    # ||o_dense - o_sparse|| <= 2 V_max (1 - Z),  Z = exp(lse_S - lse_all)
    q_lat, q_rope, kv = _rand_mla(8, B=2, T=2, H=3, L=40, dc=6, dR=2)
    B, T, H, dc = q_lat.shape
    L = kv.shape[1]
    rng = np.random.default_rng(8)
    for k in (1, 5, 20, 39):
        idx = np.stack([np.stack([np.sort(rng.choice(L, k, replace=False))
                                  for _ in range(T)]) for _ in range(B)]).astype(np.int32)
        os_, ls = orc.sparse_mla(q_lat, q_rope, kv, idx, 0.5, dc=dc)
        od, ld = orc.masked_mla(q_lat, q_rope, kv, np.ones((B, T, L), np.uint8), 0.5, dc=dc)
        vmax = np.linalg.norm(kv[..., :dc].numpy(), axis=-1).max(axis=1)  # per b
        Z = np.exp(ls - ld)
        err = np.linalg.norm(od - os_, axis=-1)
        assert np.all(err <= 2 * vmax[:, None, None] * (1 - Z) + 1e-12)


def test_output_is_linear_in_latent_values(orc):
    # with the content query zero the scores do not depend on c, and the
    # aggregation commutes with a value up-projection U_V
    rng = np.random.default_rng(9)
    L, dc, dv = 10, 4, 6
    UV = rng.standard_normal((dv, dc))
    c = rng.standard_normal((L, dc))
    kr = rng.standard_normal((L, 2))
    S = [0, 3, 7]
    o_c, _ = _mla_1q(orc, np.zeros(dc), [0.4, -1.0], c, kr, S)
    o_v, _ = _mla_1q(orc, np.zeros(dv), [0.4, -1.0], c @ UV.T, kr, S)
    np.testing.assert_allclose(UV @ o_c[0, 0, 0], o_v[0, 0, 0], rtol=1e-12, atol=1e-12)


def test_placement_invariance(orc):
    # permuting the physical cache rows and remapping the indices (same slot
    # order) leaves the output bit-identical
    q_lat, q_rope, kv = _rand_mla(10, B=1, T=2, H=2, L=25, dc=5, dR=3)
    rng = np.random.default_rng(10)
    idx = np.stack([np.sort(rng.choice(25, 8, replace=False)) for _ in range(2)])[None].astype(np.int32)
    perm = rng.permutation(25)             # new row r holds old row perm[r]
    inv = np.argsort(perm)
    kv2 = kv[:, torch.from_numpy(perm)]
    idx2 = inv[idx].astype(np.int32)
    o1, l1 = orc.sparse_mla(q_lat, q_rope, kv, idx, 0.3, dc=5)
    o2, l2 = orc.sparse_mla(q_lat, q_rope, kv2, idx2, 0.3, dc=5)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_skip_and_empty_rules(orc):
    q_lat, q_rope, kv = _rand_mla(11, B=1, T=1, H=2, L=6, dc=3, dR=2)
    a, _ = orc.sparse_mla(q_lat, q_rope, kv, np.array([[[1, 4]]], np.int32), 0.5, dc=3)
    b, _ = orc.sparse_mla(q_lat, q_rope, kv, np.array([[[-1, 1, 6, 4, 99]]], np.int32), 0.5, dc=3)
    assert np.array_equal(a, b)
    with pytest.raises(orc.OracleError):
        orc.sparse_mla(q_lat, q_rope, kv, np.array([[[-1, 7]]], np.int32), 0.5, dc=3)


def test_future_perturbation_causal_pipeline(orc):
    # indexer -> top-k -> sparse MLA on a causal prefill: changing keys and
    # values after position t leaves query t's selection and output unchanged
    from top_indexer_sparse_amd import workloads
    wl = workloads.tiny_prefill(L=40, HI=2, dI=8, topk=6, H=2, dc=4, dR=2)
    t0 = 22

    def run(w):
        s = orc.indexer(w.q_idx, w.w, w.k_idx, q_pos=w.q_pos)
        idx, cnt = orc.topk(s, w.topk, q_pos=w.q_pos)
        o, _ = orc.sparse_mla(w.q_lat, w.q_rope, w.kv, idx, w.sm_scale, dc=w.dc)
        return idx, o

    i1, o1 = run(wl)
    wl2 = workloads.DsaWorkload(**{**wl.__dict__})
    wl2.k_idx = wl.k_idx.clone()
    wl2.kv = wl.kv.clone()
    wl2.k_idx[:, t0 + 1:] = 2.0
    wl2.kv[:, t0 + 1:] *= -3.0
    i2, o2 = run(wl2)
    assert np.array_equal(i1[:, :t0 + 1], i2[:, :t0 + 1])
    assert np.array_equal(o1[:, :t0 + 1], o2[:, :t0 + 1])
    assert not np.array_equal(o1[:, t0 + 1:], o2[:, t0 + 1:])


def test_zero_fill_scatter_is_not_the_mask_form(orc):
    # A top-k implementation that writes unselected scores as 0 (instead of
    # -inf) before the softmax still gives them weight; the oracle follows the
    # mask form, so the two differ whenever some unselected weight survives.
    L = 6
    scores = np.array([2.0, -1.0, 0.5, -3.0, 1.0, -2.0])
    vals = np.array([1.0, 2.0, 3.0, 4.0, 5.0, 6.0])
    c, kr = _scalar_rows(vals, scores)
    S = [0, 2, 4]
    ours, _ = _mla_1q(orc, [0.0], [1.0], c, kr, S)
    zeroed = np.where(np.isin(np.arange(L), S), scores, 0.0)
    wz = np.exp(zeroed) / np.exp(zeroed).sum()
    assert abs(float(wz @ vals) - ours[0, 0, 0, 0]) > 0.1


# --------------------------------------------------------------------------
# block-sparse decode (GQA), block toy and pooling
# --------------------------------------------------------------------------

def test_block_pool_closed_forms(orc):
    B, L, Hkv, d, blk = 1, 12, 2, 3, 4
    ramp = torch.arange(L, dtype=torch.float64)[None, :, None, None].expand(B, L, Hkv, d).contiguous()
    rep = orc.block_pool(ramp, blk)
    # mean of n*4 .. n*4+3 is n*4 + 1.5
    for n in range(3):
        assert np.all(rep[0, n] == n * 4 + 1.5)
    # incomplete tail block is not pooled
    assert orc.block_pool(ramp[:, :11].contiguous(), blk).shape[1] == 2


def _sdpa_masked(q, k, v, mask, scale):
    # q [Hq,d]; k,v [L,Hkv,d]; mask [Hq, L] bool (true = visible)
    Hq = q.shape[0]
    Hkv = k.shape[1]
    g = Hq // Hkv
    kk = k.permute(1, 0, 2).repeat_interleave(g, 0)    # [Hq,L,d]
    vv = v.permute(1, 0, 2).repeat_interleave(g, 0)
    out = torch.nn.functional.scaled_dot_product_attention(
        q[:, None], kk, vv, attn_mask=mask[:, None], scale=scale)
    return out[:, 0].numpy()


def test_block_toy_page_example(orc, ex):
    e = ex["block_toy"]
    g = torch.Generator().manual_seed(12)
    n, blk, d = e["n"], e["block"], 8
    k = torch.randn(1, n, 1, d, generator=g, dtype=torch.float64)
    v = torch.randn(1, n, 1, d, generator=g, dtype=torch.float64)
    # make blocks 0 and 1 the best-scoring representatives for the query
    q = torch.randn(1, 1, d, generator=g, dtype=torch.float64)
    k[0, :8, 0] += 3.0 * q[0, 0] / q[0, 0].norm()
    k[0, 8:, 0] -= 3.0 * q[0, 0] / q[0, 0].norm()
    out, blocks = orc.block_sparse_decode(q, k, v, blk, 2, 0, 0, d ** -0.5)
    assert blocks[0, 0].tolist() == e["selected_blocks"]
    mask = torch.zeros(1, n, dtype=torch.bool)
    mask[0, e["tokens_read"]] = True
    ref = _sdpa_masked(q[0], k[0], v[0], mask, d ** -0.5)
    np.testing.assert_allclose(out[0], ref, rtol=1e-12, atol=1e-12)


def test_block_sparse_union_sink_window_gqa(orc):
    g = torch.Generator().manual_seed(13)
    B, L, Hq, Hkv, d, blk = 2, 64, 4, 2, 8, 8
    q = torch.randn(B, Hq, d, generator=g, dtype=torch.float64)
    k = torch.randn(B, L, Hkv, d, generator=g, dtype=torch.float64)
    v = torch.randn(B, L, Hkv, d, generator=g, dtype=torch.float64)
    nsel, n_sink, n_win = 2, 3, 10
    out, blocks = orc.block_sparse_decode(q, k, v, blk, nsel, n_sink, n_win, 0.3)
    rep = orc.block_pool(k, blk)
    for b in range(B):
        mask = torch.zeros(Hq, L, dtype=torch.bool)
        for h in range(Hq):
            gh = h // (Hq // Hkv)
            sc = rep[b, :, gh] @ q[b, h].numpy()
            order = sorted(range(L // blk), key=lambda i: (-sc[i], i))[:nsel]
            assert blocks[b, h].tolist() == sorted(order)
            for bi in order:
                mask[h, bi * blk:(bi + 1) * blk] = True
            mask[h, :n_sink] = True
            mask[h, L - n_win:] = True
        ref = _sdpa_masked(q[b], k[b], v[b], mask, 0.3)
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-12)


def test_block_sparse_all_blocks_is_dense(orc):
    g = torch.Generator().manual_seed(14)
    B, L, Hq, Hkv, d, blk = 1, 32, 2, 1, 4, 8
    q = torch.randn(B, Hq, d, generator=g, dtype=torch.float64)
    k = torch.randn(B, L, Hkv, d, generator=g, dtype=torch.float64)
    v = torch.randn(B, L, Hkv, d, generator=g, dtype=torch.float64)
    out, _ = orc.block_sparse_decode(q, k, v, blk, L // blk, 0, 0, 0.5)
    ref = _sdpa_masked(q[0], k[0], v[0], torch.ones(Hq, L, dtype=torch.bool), 0.5)
    np.testing.assert_allclose(out[0], ref, rtol=1e-12, atol=1e-12)


def test_block_sparse_given_blocks_reproduces_own_choice(orc):
    # passing the oracle's own choice back in gives the same output, bit for
    # bit, and echoes the same blocks (per head and with a shared choice)
    g = torch.Generator().manual_seed(18)
    B, L, Hq, Hkv, d, blk = 2, 100, 4, 2, 8, 8
    q = torch.randn(B, Hq, d, generator=g, dtype=torch.float64)
    k = torch.randn(B, L, Hkv, d, generator=g, dtype=torch.float64)
    v = torch.randn(B, L, Hkv, d, generator=g, dtype=torch.float64)
    for shared in (False, True):
        out, blocks = orc.block_sparse_decode(q, k, v, blk, 3, 2, 7, 0.35, shared=shared)
        o2, b2 = orc.block_sparse_decode(q, k, v, blk, 3, 2, 7, 0.35, given_blocks=blocks)
        np.testing.assert_array_equal(b2, blocks)
        np.testing.assert_array_equal(o2, out)


def test_block_sparse_given_blocks_is_masked_softmax(orc):
    # an arbitrary given choice (not the top blocks; with a duplicate, an
    # out-of-range entry and -1 padding) attends over exactly the union of
    # those blocks, the sinks and the window: torch SDPA with that mask
    g = torch.Generator().manual_seed(19)
    B, L, Hq, Hkv, d, blk = 1, 70, 2, 1, 8, 8   # 8 complete blocks, ragged tail
    q = torch.randn(B, Hq, d, generator=g, dtype=torch.float64)
    k = torch.randn(B, L, Hkv, d, generator=g, dtype=torch.float64)
    v = torch.randn(B, L, Hkv, d, generator=g, dtype=torch.float64)
    given = np.array([[[5, 1, 5, -1], [8, 0, 3, 7]]], dtype=np.int32)  # 8 is past the blocks
    out, blocks = orc.block_sparse_decode(q, k, v, blk, 4, 2, 3, 0.5, given_blocks=given)
    assert blocks[0, 0].tolist()[:2] == [1, 5] and blocks[0, 1].tolist()[:3] == [0, 3, 7]
    mask = torch.zeros(Hq, L, dtype=torch.bool)
    for h, bl in ((0, [1, 5]), (1, [0, 3, 7])):
        for bi in bl:
            mask[h, bi * blk:(bi + 1) * blk] = True
    mask[:, :2] = True
    mask[:, L - 3:] = True
    ref = _sdpa_masked(q[0], k[0], v[0], mask, 0.5)
    np.testing.assert_allclose(out[0], ref, rtol=1e-12, atol=1e-12)


def test_block_sparse_empty_visible_set(orc):
    # L < blk, no sinks, no window: nothing is visible; out = 0 when allowed
    g = torch.Generator().manual_seed(20)
    q = torch.randn(1, 2, 4, generator=g, dtype=torch.float64)
    k = torch.randn(1, 5, 1, 4, generator=g, dtype=torch.float64)
    v = torch.randn(1, 5, 1, 4, generator=g, dtype=torch.float64)
    with pytest.raises(orc.OracleError):
        orc.block_sparse_decode(q, k, v, 8, 2, 0, 0, 0.5)
    out, blocks = orc.block_sparse_decode(q, k, v, 8, 2, 0, 0, 0.5, allow_empty=True)
    assert np.all(out == 0) and np.all(blocks == -1)


# --------------------------------------------------------------------------
# GQA-shared block choice (the group's heads share one block set)
# --------------------------------------------------------------------------

def test_gqa_shared_choice_page_example(orc, ex):
    # two heads over three blocks; block keys are unit vectors, so each head's
    # block scores are exactly the page's numbers
    e = ex["gqa_shared_choice"]
    sc = torch.tensor(e["head_scores"], dtype=torch.float64)  # [2 heads, 3 blocks]
    Hq, nblk = sc.shape
    q = sc[None].clone()                                       # [1, 2, d=3]
    k = torch.eye(nblk, dtype=torch.float64)[None, :, None, :]  # blk = 1: krep = k
    g = torch.Generator().manual_seed(15)
    v = torch.randn(1, nblk, 1, nblk, generator=g, dtype=torch.float64)
    _, own = orc.block_sparse_decode(q, k, v, 1, 1, 0, 0, 1.0)
    assert own[0, :, 0].tolist() == e["per_head_top1"]
    out, shared = orc.block_sparse_decode(q, k, v, 1, 1, 0, 0, 1.0, shared=True)
    assert shared[0, :, 0].tolist() == e["group_top1"] * Hq
    # one visible token: the output is its value row
    for h in range(Hq):
        np.testing.assert_array_equal(out[0, h], v[0, e["group_top1"][0], 0].numpy())


def test_gqa_shared_choice_sums_group_scores(orc):
    g = torch.Generator().manual_seed(16)
    B, L, Hq, Hkv, d, blk = 2, 96, 8, 2, 8, 8
    q = torch.randn(B, Hq, d, generator=g, dtype=torch.float64)
    k = torch.randn(B, L, Hkv, d, generator=g, dtype=torch.float64)
    v = torch.randn(B, L, Hkv, d, generator=g, dtype=torch.float64)
    nsel, n_sink, n_win = 3, 2, 5
    out, blocks = orc.block_sparse_decode(q, k, v, blk, nsel, n_sink, n_win, 0.4, shared=True)
    rep = orc.block_pool(k, blk)
    G = Hq // Hkv
    for b in range(B):
        mask = torch.zeros(Hq, L, dtype=torch.bool)
        for h in range(Hq):
            gh = h // G
            tot = sum(rep[b, :, gh] @ q[b, hh].numpy() for hh in range(gh * G, gh * G + G))
            order = sorted(range(L // blk), key=lambda i: (-tot[i], i))[:nsel]
            assert blocks[b, h].tolist() == sorted(order)
            for bi in order:
                mask[h, bi * blk:(bi + 1) * blk] = True
            mask[h, :n_sink] = True
            mask[h, L - n_win:] = True
        ref = _sdpa_masked(q[b], k[b], v[b], mask, 0.4)
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-12)


def test_gqa_shared_choice_group_of_one_is_per_head(orc):
    g = torch.Generator().manual_seed(17)
    B, L, H, d, blk = 1, 64, 3, 4, 8
    q = torch.randn(B, H, d, generator=g, dtype=torch.float64)
    k = torch.randn(B, L, H, d, generator=g, dtype=torch.float64)
    v = torch.randn(B, L, H, d, generator=g, dtype=torch.float64)
    o1, b1 = orc.block_sparse_decode(q, k, v, blk, 2, 1, 4, 0.5)
    o2, b2 = orc.block_sparse_decode(q, k, v, blk, 2, 1, 4, 0.5, shared=True)
    assert np.array_equal(b1, b2)
    np.testing.assert_array_equal(o1, o2)


# --------------------------------------------------------------------------
# selection over compressed entries (CSA-style): indexer + top-k over the
# entries, MQA core attention with keys = values = entries, plus a window
# --------------------------------------------------------------------------

def _csa_inputs(seed, B=2, Lc=40, HI=3, dI=8, H=4, c=16, n_win=5):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=g, dtype=torch.float64)
    return (r(B, HI, dI), torch.rand(B, HI, generator=g, dtype=torch.float64), r(B, Lc, dI),
            r(B, H, c), r(B, Lc, c), r(B, n_win, c) if n_win else None)


def _softmax_attn(q, rows, scale):
    # q [H,c], rows [n,c] (keys = values) -> out [H,c], lse [H]
    z = q @ rows.T * scale
    m = z.max(dim=1, keepdim=True).values
    p = torch.exp(z - m)
    return (p @ rows / p.sum(dim=1, keepdim=True)).numpy(), (m[:, 0] + torch.log(p.sum(dim=1))).numpy()


def test_csa_all_entries_no_window_is_dense_mqa(orc):
    # k >= Lc and no window: every entry is attended, keys = values
    qi, w, ki, q, comp, _ = _csa_inputs(20, n_win=0)
    out, lse, idx, cnt = orc.csa_decode(qi, w, ki, q, comp, None, 64, 0.25)
    assert np.all(cnt == 40) and np.all(idx[:, :40] == np.arange(40)) and np.all(idx[:, 40:] == -1)
    for b in range(2):
        ro, rl = _softmax_attn(q[b], comp[b], 0.25)
        np.testing.assert_allclose(out[b], ro, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[b], rl, rtol=1e-12, atol=1e-12)


def test_csa_union_is_the_log_sum_exp_merge_of_both_branches(orc):
    # one softmax over selected entries and window entries equals merging the
    # two branches' outputs by their log-sum-exp weights
    qi, w, ki, q, comp, win = _csa_inputs(21)
    k = 7
    out, lse, idx, cnt = orc.csa_decode(qi, w, ki, q, comp, win, k, 0.3)
    for b in range(2):
        sel = comp[b][torch.as_tensor(idx[b, :cnt[b]], dtype=torch.long)]
        os_, ls = _softmax_attn(q[b], sel, 0.3)
        ow, lw = _softmax_attn(q[b], win[b], 0.3)
        a, c2 = np.exp(ls - np.maximum(ls, lw)), np.exp(lw - np.maximum(ls, lw))
        merged = (a[:, None] * os_ + c2[:, None] * ow) / (a + c2)[:, None]
        np.testing.assert_allclose(out[b], merged, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse[b], np.maximum(ls, lw) + np.log(a + c2), rtol=1e-12)


def test_csa_selection_is_the_indexer_top_k(orc):
    # the selected entries are the k highest index scores (brute force), and an
    # entry outside the selection and the window does not move the output
    qi, w, ki, q, comp, win = _csa_inputs(22)
    k = 6
    out, _, idx, cnt = orc.csa_decode(qi, w, ki, q, comp, win, k, 0.3)
    for b in range(2):
        sc = [sum(float(w[b, h]) * max(0.0, float(qi[b, h] @ ki[b, s])) for h in range(3))
              for s in range(40)]
        assert sorted(idx[b, :k].tolist()) == sorted(sorted(range(40), key=lambda s: (-sc[s], s))[:k])
    unsel = [s for s in range(40) if s not in idx[1, :k]][0]
    comp2 = comp.clone()
    comp2[1, unsel] += 5.0
    out2, _, _, _ = orc.csa_decode(qi, w, ki, q, comp2, win, k, 0.3)
    np.testing.assert_array_equal(out2, out)
    win2 = win.clone()
    win2[1, 0] += 1.0
    out3, _, _, _ = orc.csa_decode(qi, w, ki, q, comp, win2, k, 0.3)
    assert np.abs(out3[1] - out[1]).max() > 1e-3 and np.array_equal(out3[0], out[0])
